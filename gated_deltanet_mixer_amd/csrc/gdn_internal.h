// gdn_internal.h -- launchers behind the C ABI (host side, not exported).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// g and beta hold the gate logits a and b when A_log and dt_bias are set.
constexpr int kMaxDecodeTokens = 8;  // tokens per sequence of one decode call

struct DecodeParams {
    const uint16_t *q, *k, *v, *z, *conv_w, *norm_w;
    const float *g, *beta, *A_log, *dt_bias;
    float *state;
    uint16_t *conv_state, *o;
    float *state_snaps;    // [T-1][B][Hv][128][128] or nullptr
    uint16_t *conv_snaps;  // [T-1][B][3][Cc] or nullptr
    int B, T, Hk, Hv, conv_width, norm;  // T: tokens per sequence, 1..8
    float eps_l2, eps_norm;
};

struct PrefillParams {
    const uint16_t *q, *k, *v, *z, *conv_w, *norm_w, *conv_state_in;
    const float *g, *beta, *A_log, *dt_bias, *state_in;
    uint16_t *o, *conv_state_out;
    float *state_out;
    void *workspace;
    const int *cu_seqlens;  // packed sequences: [B + 1] token offsets into [T] rows; nullptr: B rows of T
    int B, T, Hk, Hv, conv_width, norm;
    float eps_l2, eps_norm;
};

// Value-dimension slicing and workspace layout chosen for a prefill shape.
// The workspace starts with the exchange area (its first 32-bit word is the error word),
// which the prep kernel clears at the start of every call; the operand blocks follow.
struct PrefillPlan {
    int nt;              // 16-column value tiles per sequential-pass workgroup: 1 or 2
    int bv;              // value columns per sequential-pass workgroup (16 * nt)
    int nslice;          // workgroups per (sequence, value head): 128 / bv
    int nchunks;         // ceil(T / 64)
    long long nslots;    // chunk operand slots: B nchunks, or floor(T / 64) + B for packed sequences
    size_t xch_bytes;    // exchange area: 256-byte header (error word, queue tickets, exit count),
                         // then the tagged per-row partial sums of every (sequence, value head)
    size_t mbox_bytes;   // the tagged partial sums inside the exchange area
    size_t qk_bytes;     // per (slot, key head): q^, k^, k^T fragments (fp16)
    size_t tp_bytes;     // per (slot, value head): T diag(beta), P (lower blocks, fp16), decay vectors
    int nseg;            // segments per sequence of the two-level scan (1: the plain sequential pass)
    int seg_chunks;      // chunks per segment
    size_t seg_out_bytes, seg_state_bytes, seg_frag_bytes;  // two-level scan: read-outs, segment maps, start states
    size_t total_bytes;
};

// Where each region of a prefill workspace lies.
struct PrefillRegions {
    unsigned int *err;       // error word: bit 0 a bounded wait timed out, bit 1 a packed sequence was skipped
    unsigned int *tickets;   // [8] work-queue tickets
    unsigned int *exits;     // workgroups that left the two-level scan's first pass
    unsigned long long *mbox;
    _Float16 *qkf, *tpf;
    unsigned char *seg;      // two-level scan regions (read-outs, segment maps, start states)
};

// Byte offsets inside the header of the exchange area.
constexpr size_t kErrOffset = 0, kTicketOffset = 64, kExitOffset = 128, kHeaderBytes = 256;

// Record why a launch failed, for gdn_last_error() on the calling thread;
// both return -1 so a launcher can `return fail(...)`.
int fail(const char *what, hipError_t e);
int fail(const char *what);

// segments: 0 lets the plan choose, 1 keeps the plain sequential pass, n >= 2 asks for n
// segments of the two-level scan (even batches only).
int plan_prefill(int B, int T, int Hk, int Hv, bool packed, int segments, PrefillPlan *plan);
PrefillRegions prefill_regions(void *workspace, const PrefillPlan &plan, int B, int Hv);
int launch_decode(const DecodeParams &p, hipStream_t stream);
size_t decode_lds_bytes(int T, int r);  // LDS of one decode workgroup
int launch_prefill(const PrefillParams &p, const PrefillPlan &plan, hipStream_t stream);
int launch_pass(const PrefillParams &p, const PrefillPlan &plan, const PrefillRegions &rg, hipStream_t stream);
int launch_state_init(float *state, size_t n_state, uint16_t *conv_state, size_t n_conv,
                      hipStream_t stream);

} // namespace gdn
