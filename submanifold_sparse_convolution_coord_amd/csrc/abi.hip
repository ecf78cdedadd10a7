// Library-wide entry points of the C ABI: version, status text and the digest of the sources
// the library was built from.
#include <hip/hip_runtime.h>

#include "common.h"

#ifndef SSC_SOURCE_DIGEST
#define SSC_SOURCE_DIGEST "unknown"
#endif

extern "C" int ssc_version(void) { return 200; }

extern "C" const char* ssc_source_digest(void) { return SSC_SOURCE_DIGEST; }

extern "C" const char* ssc_status_string(int status) {
  switch (status) {
    case SSC_OK: return "ok";
    case SSC_ERR_ARG: return "invalid argument (null, negative size, bad dtype or misaligned)";
    case SSC_ERR_COORD_RANGE: return "coordinate outside [0,batch) x [0,grid)";
    case SSC_ERR_DUPLICATE: return "duplicate coordinate";
    case SSC_ERR_UNSUPPORTED: return "unsupported shape";
    case SSC_ERR_WORKSPACE: return "workspace or plan buffer too small";
    case SSC_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}
