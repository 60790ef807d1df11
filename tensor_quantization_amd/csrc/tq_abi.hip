// tq_abi.hip -- ABI utilities: version, status names, default code ranges.
#include "tq_host.h"

extern "C" {

int tq_abi_version(void) { return 1; }

const char* tq_status_str(int status)
{
    switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_ALIGN: return "misaligned pointer";
    case TQ_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
    }
}

// default_q_range (docs.rs baracuda_kernels::quantize, function
// default_q_range): S8 [-128, 127], U8 [0, 255]; 4-bit widths alongside;
// symmetric mode uses [-qmax, qmax].
tq_status tq_default_q_range(int code, int symmetric, int32_t* host_qmin, int32_t* host_qmax)
{
    if (!host_qmin || !host_qmax) return TQ_ERR_INVALID;
    switch (code) {
    case TQ_S8: *host_qmin = symmetric ? -127 : -128; *host_qmax = 127; return TQ_OK;
    case TQ_S4: *host_qmin = symmetric ? -7 : -8; *host_qmax = 7; return TQ_OK;
    case TQ_U8: if (symmetric) return TQ_ERR_INVALID; *host_qmin = 0; *host_qmax = 255; return TQ_OK;
    case TQ_U4: if (symmetric) return TQ_ERR_INVALID; *host_qmin = 0; *host_qmax = 15; return TQ_OK;
    default: return TQ_ERR_INVALID;
    }
}

}  // extern "C"
