#include "common.h"
#include "../launch.h"
namespace hypic {
hipError_t launch_seam(int, int, bool, const SeamArgs&, hipStream_t) { return hipErrorInvalidValue; }
}
