#include "m3_internal.h"
namespace m3 {
bool scan_mfma_supported(const ScanArgs&) { return false; }
size_t scan_mfma_workspace_bytes(const ScanArgs&) { return 0; }
hipError_t launch_scan_mfma(const ScanArgs&, hipStream_t) { return hipErrorInvalidValue; }
}
