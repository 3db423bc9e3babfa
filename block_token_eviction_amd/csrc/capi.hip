// Library-wide C-ABI entry points of libbte: status strings and version.
#include "bte.h"

extern "C" const char* bte_status_string(int status) {
  switch (status) {
    case BTE_OK: return "ok";
    case BTE_ERR_NULL: return "a required pointer is NULL";
    case BTE_ERR_DIM: return "a size is out of range or inconsistent";
    case BTE_ERR_UNSUPPORTED: return "unsupported head_dim, block, pool kernel, row size or dtype";
    case BTE_ERR_ALIGN: return "a pointer or row size breaks the alignment rule";
    case BTE_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    default: return "unknown status";
  }
}

extern "C" int bte_version(void) { return 100; }
