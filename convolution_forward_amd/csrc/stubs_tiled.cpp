// Placeholders for the tiled kernel families until they are built.
#include "internal.h"

namespace convfwd {

bool dense_tiled_supports(const DenseProblem &) { return false; }
hipError_t launch_dense_tiled(const DenseProblem &, hipStream_t) { return hipErrorNotSupported; }
bool dw_tiled_supports(const DwProblem &) { return false; }
hipError_t launch_dw_tiled(const DwProblem &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace convfwd
