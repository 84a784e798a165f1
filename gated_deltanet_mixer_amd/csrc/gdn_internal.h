// gdn_internal.h -- launchers behind the C ABI (host side, not exported).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct DecodeParams {
    const uint16_t *q, *k, *v, *z, *conv_w, *norm_w;
    const float *g, *beta;
    float *state;
    uint16_t *conv_state, *o;
    int B, Hk, Hv, conv_width, norm;
    float eps_l2, eps_norm;
};

struct PrefillParams {
    const uint16_t *q, *k, *v, *z, *conv_w, *norm_w, *conv_state_in;
    const float *g, *beta, *state_in;
    uint16_t *o, *conv_state_out;
    float *state_out;
    void *workspace;
    int B, T, Hk, Hv, conv_width, norm;
    float eps_l2, eps_norm;
};

// Value-dimension slicing chosen for a prefill shape (columns per workgroup).
struct PrefillPlan {
    int bv;          // 16, 32 or 64 value columns per workgroup
    int nslice;      // 128 / bv
    size_t qk_bytes;     // fp16 normalised q/k operands
    size_t mbox_bytes;   // exchange area (tagged partial sums, counters, error word)
};

int plan_prefill(int B, int T, int Hk, int Hv, PrefillPlan *plan);
int launch_decode(const DecodeParams &p, hipStream_t stream);
int launch_prefill(const PrefillParams &p, const PrefillPlan &plan, hipStream_t stream);
int launch_state_init(float *state, size_t n_state, uint16_t *conv_state, size_t n_conv,
                      hipStream_t stream);

} // namespace gdn
