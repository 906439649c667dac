// Library identity and status strings of the treeverify C ABI.
#include <string.h>

#include "tv_internal.h"

TV_API int tv_abi_version(void) { return TV_ABI_VERSION; }

TV_API const char* tv_status_string(tv_status s) {
  // a C caller may pass any int here: read the argument's bits as an int, never as an
  // enum value outside the enumeration
  int v;
  memcpy(&v, &s, sizeof v);
  switch (v) {
    case TV_OK: return "ok";
    case TV_ERR_NULL: return "a required pointer is NULL";
    case TV_ERR_SHAPE: return "a size argument is out of range or inconsistent";
    case TV_ERR_DTYPE: return "unknown dtype";
    case TV_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or pointer alignment";
    case TV_ERR_WORKSPACE: return "workspace missing or too small";
    case TV_ERR_HIP: return "HIP runtime error at launch";
  }
  return "unknown status";
}
