// api.hip -- library-wide entry points of libbi.so (version and status names).
#include "common.h"

extern "C" int bi_abi_version(void) { return BI_ABI_VERSION; }

extern "C" const char *bi_status_str(int status) {
  switch (status) {
    case BI_OK: return "BI_OK";
    case BI_ERR_NULL: return "BI_ERR_NULL: a required pointer is NULL";
    case BI_ERR_SHAPE: return "BI_ERR_SHAPE: a size or stride is out of range or not supported";
    case BI_ERR_ALIGN: return "BI_ERR_ALIGN: a pointer or stride is not aligned";
    case BI_ERR_WORKSPACE: return "BI_ERR_WORKSPACE: split-K workspace missing or too small";
    case BI_ERR_ALIAS: return "BI_ERR_ALIAS: an output overlaps another tensor";
    case BI_ERR_HIP: return "BI_ERR_HIP: the HIP runtime reported an error";
    case BI_ERR_UNSUPPORTED: return "BI_ERR_UNSUPPORTED: not implemented by the library";
    default: return "unknown bi_status";
  }
}
