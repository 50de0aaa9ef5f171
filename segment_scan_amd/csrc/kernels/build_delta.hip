#include "common.h"
#include "../launch.h"
namespace hypic {
hipError_t launch_build_delta(int, bool, const BuildArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
}
