// noalloc.hip -- sla_forward_noalloc: the forward pass with its scratch
// memory in a static device array instead of a caller-provided workspace,
// for callers that cannot allocate (code under graph capture, serving loops
// that forbid hipMalloc).
//
// The array `scratch` is a file-scope __device__ object: every GPU the
// library runs on holds its own copy, at its own address, from the moment
// the code object is loaded on that device until the process ends.  In host
// code the name `scratch` is only a host-side stand-in for that object, so
// host code never passes it to a kernel or a copy: on the first call on a
// device (with that device current) its device address is looked up once
// with hipGetSymbolAddress and kept per device; every later call passes that
// address as the workspace of sla_forward, whose kernels take it as an
// argument like any workspace.
//
// The forward pass reads nothing from its workspace before writing it (its
// contents on entry do not matter), so nothing is cleared between calls.
// Calls that overlap on one GPU (two streams, or two host threads) share the
// one array and race; callers serialise them.
#include <mutex>

#include "sla.h"
#include "sla_launch.h"

static __device__ __align__(256) unsigned char scratch[SLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t SCRATCH_BYTES = SLA_NOALLOC_SCRATCH_BYTES;
constexpr int MAX_DEVICES = 64;

std::mutex g_mu;
void *g_scratch[MAX_DEVICES];   // device address of `scratch`, per device; null until looked up

// The device address of this device's copy of `scratch`, looked up on first use.
hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

sla_status sla_forward_noalloc(const void *q, const void *k, const void *v, const float *w_proj, sla_dtype in_dtype,
                               sla_dtype out_dtype, int B, int H, int N, int d, int block, double crit_frac,
                               double negl_frac, sla_phi phi, void *out, int8_t *mask_out, void *stream) {
    // everything is checked on the host before the first device call
    if (!q || !k || !v || !w_proj || !out) return sla::set_error(SLA_ERR_INVALID_ARG, "null tensor pointer");
    if (phi != SLA_PHI_SOFTMAX) return sla::set_error(SLA_ERR_UNSUPPORTED, "feature map %d not supported", (int)phi);
    if (out_dtype != SLA_F32 && out_dtype != in_dtype)
        return sla::set_error(SLA_ERR_UNSUPPORTED, "output dtype must be F32 or the input dtype");
    size_t need = 0;
    // shape, dtype and fraction errors come back from here with their message
    sla_status st = sla_workspace_size(B, H, N, d, block, in_dtype, crit_frac, negl_frac, &need);
    if (st != SLA_OK) return st;
    if (need > SCRATCH_BYTES)
        return sla::set_error(SLA_ERR_WORKSPACE,
                              "these sizes need %zu bytes of scratch; the static scratch of sla_forward_noalloc "
                              "holds %zu (use sla_forward with a workspace)",
                              need, SCRATCH_BYTES);
    void *ws = nullptr;
    hipError_t e = scratch_address(&ws);
    if (e != hipSuccess)
        return sla::set_error(SLA_ERR_DEVICE, "hipGetSymbolAddress of the static scratch: %s", hipGetErrorString(e));
    return sla_forward(q, k, v, w_proj, in_dtype, out_dtype, B, H, N, d, block, crit_frac, negl_frac, phi, out,
                       mask_out, ws, SCRATCH_BYTES, stream);
}

}  // extern "C"
