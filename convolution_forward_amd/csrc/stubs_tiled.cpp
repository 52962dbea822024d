// Placeholders for the tiled kernel families until they are built.
#include "internal.h"

namespace convfwd {

bool dw_tiled_supports(const DwProblem &) { return false; }
hipError_t launch_dw_tiled(const DwProblem &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace convfwd
