// gdn_prefill_common.h -- layout of the prefill workspace and device helpers shared by
// the chunk-prep kernel and the sequential-pass kernels (internal; not part of the ABI).
#pragma once
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int kD = 128;        // head width
constexpr int kC = 64;         // chunk length
constexpr int kTiles = 8;      // 16-column tiles per head
constexpr int kMboxRing = 8;   // gated-norm mailbox slots per (head, 16-column tile)
constexpr uint32_t kSpinLimit = 1u << 20;  // bound of every cross-workgroup wait (~0.3 s)

// LDS pitches (elements) so that 16-row MFMA fragment reads hit distinct banks.
constexpr int P128 = kD + 8;   // fp16 rows of 128
constexpr int P64 = kC + 8;    // fp16 rows of 64
constexpr int PL = kC + 4;     // fp32 rows of 64
constexpr int PTD = 20;        // fp32 rows of a 16x16 block

// conv(v) of a slice in the sequential pass, fp16 column-major: column j starts at
// vcol(j).  The 136-byte stride puts the 16 columns that one X read covers (8 bytes per
// lane) on distinct LDS banks; the 16-byte shift of columns 16..31 does the same for the
// lanes of a conv store, 8 column groups by the row groups of a half-wave.  (The segment
// pass keeps P64 columns and plain output rows: there the same change measured no gain.)
constexpr int kVStride = kC + 4;
__host__ __device__ constexpr int vcol(int j) { return j * kVStride + 8 * ((j >> 4) & 1); }
__host__ __device__ constexpr int vtile(int bv) { return bv * kVStride + 8; }  // fp16 of one buffer
// Pre-norm output ring of the sequential pass, fp32 column-major [bv][PL]: row i of column j sits
// at orow(bv, i, j).  The gating lanes read one 8-column group of one row each, a half-wave
// covering 256 / bv consecutive rows; unrotated, the groups of a row fall on one bank, rotated
// by 256 / bv rows per group they fill all 32.  Rows 4 m .. 4 m + 3 stay together, so a float4
// of 4 rows is still one 16-byte store.
__host__ __device__ constexpr int orot(int bv) { return 256 / bv; }
__host__ __device__ constexpr int orow(int bv, int i, int j) { return (i + (j >> 3) * orot(bv)) & (kC - 1); }

// Workspace blocks (fp16 elements), written by the prep kernel as MFMA operand
// fragments: fragment f holds, for lane L = l16 + 16 lq, the 8 values of row
// (tile row) + l16 at contraction indices 32 ks + {4 lq .. 4 lq + 3} and
// 32 ks + 16 + {4 lq .. 4 lq + 3} -- the rows of two adjacent 16-row
// accumulator tiles as they sit in one lane.
//   per (sequence, chunk, key head), kQKF:  q^ f = 0..15 and k^ f = 16..31 (row tile f>>2,
//                                           k-step f&3 over keys), then k^T f = 32..47
//                                           (key-row tile (f-32)>>1, token k-step
//                                           (f-32)&1: the A operand of K^T Delta)
//   per (sequence, chunk, value head), kTPF: T diag(beta) f = 0..5 (lower-triangular 64x64,
//                                           only the blocks that are not all zero), fp32
//                                           e^{G_i} [64], e^{G_C - G_i} [64], e^{G_C} [4]
//                                           (1 KB), then P = (Q K^T) o R f = 0..5
constexpr int kTBS = 20;                               // fp16 row pitch of a staged 16x16 block: the 16 rows
                                                       // of one 8-byte fragment read fall on distinct banks
constexpr int kBlk = 16 * kTBS;                        // one staged 16x16 block (prep)
constexpr int kFrag = 64 * 8;                          // one fragment: 64 lanes x 8 fp16
constexpr int kQKF = 48 * kFrag;
constexpr int kKOff = 16 * kFrag;                      // k^ fragments inside a q/k block
constexpr int kKTOff = 32 * kFrag;                     // k^T fragments inside a q/k block
constexpr int kVecOff = 6 * kFrag;
constexpr int kPOff = kVecOff + 512;                   // after 256 fp32
constexpr int kTPF = kPOff + 6 * kFrag;

__host__ __device__ constexpr int kpos(int m) { return m < 4 ? 8 * m : 8 * (m - 4) + 4; }


__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Accumulator tiles a (rows 4q..4q+3 of a 16-row tile) and b (the next tile)
// as one 8-element MFMA B operand, in the permuted k order described above.
__device__ __forceinline__ half8 pack_tiles(const floatx4 &a, const floatx4 &b) {
    return half8{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3],
                 (_Float16)b[0], (_Float16)b[1], (_Float16)b[2], (_Float16)b[3]};
}

#define GDN_AS1 __attribute__((address_space(1)))
#define GDN_AS3 __attribute__((address_space(3)))

// 16 bytes per lane from global memory (lane address) into LDS at dst + 16 lane
__device__ __forceinline__ void dma16(const void *src_lane, void *dst_wave) {
    __builtin_amdgcn_global_load_lds((const GDN_AS1 void *)src_lane, (GDN_AS3 void *)dst_wave, 16, 0, 0);
}
// the same through a buffer resource: lanes past the resource read as zero
__device__ __forceinline__ void dma16b(__amdgpu_buffer_rsrc_t r, int voff, void *dst_wave) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (GDN_AS3 void *)dst_wave, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, unsigned int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ half8 ld_frag(__amdgpu_buffer_rsrc_t r, int voff, int f) {
    return __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, f * 1024, 0));
}
__device__ __forceinline__ float4 ld_f4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const floatx4 v = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    return make_float4(v[0], v[1], v[2], v[3]);
}
// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// A 16-byte or 4-byte store into the workspace through a buffer resource.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_ws(__amdgpu_buffer_rsrc_t r, int voff, half8 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, 0, 0);
}
__device__ __forceinline__ void st_ws(__amdgpu_buffer_rsrc_t r, int voff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, 0, 0);
}
// 4 fp16 from LDS through the transposing read: within each 16-lane group the
// lanes' 8-byte chunks form a 4 x 16 matrix (row = lane / 4, column = 4 (lane % 4)
// + element) and lane i receives column i.
__device__ __forceinline__ half4 lds_tr16(const _Float16 *p) {
    typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4s;
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDN_AS3 v4s *)(p));
    return __builtin_bit_cast(half4, r);
}

// ========================================================================
// chunk_prep_kernel
// ========================================================================

// Where sequence b's tokens and chunk operands sit.  An even batch (cu == nullptr):
// tokens b T .. b T + T - 1 and operand slots b nch .. b nch + nch - 1.  Packed
// sequences: tokens cu[b] .. cu[b+1] - 1 and slots from floor(cu[b] / 64) + b on.
// Those bases grow from one sequence to the next by at least the chunk count of
// the earlier one, so the slot ranges never overlap and all of them lie below
// floor(T / 64) + B, without a prefix sum over the chunk counts.  Chunks start at
// each sequence's first token: the recurrent state and the conv window start
// afresh at every sequence boundary.  A packed sequence whose bounds are not
// 0 <= cu[b] < cu[b+1] <= T comes back with no chunks (and nothing is read or
// written for it); so does every sequence when the offsets are not non-decreasing
// from cu[0] to cu[B] (the slot ranges, and the search that maps a slot to its
// sequence, rely on that order).
struct SeqInfo {
    size_t tok0;
    int T, c0, nch;
};
// Whether cu[0..B] is non-decreasing, tested by the calling wave (every lane of it
// takes part; the result is wave-uniform).
__device__ __forceinline__ bool cu_ordered(const int *cu, int B) {
    const int lane = threadIdx.x & 63;
    bool bad = false;
    for (int j = lane; j < B; j += 64) bad = bad || cu[j] > cu[j + 1];
    return __ballot(bad) == 0;
}
// Called by whole waves (cu_ordered needs every lane).
__device__ __forceinline__ SeqInfo seq_info(const int *cu, int b, int T, int nch, int B) {
    if (!cu) return SeqInfo{(size_t)b * T, T, b * nch, nch};
    const int t0 = cu[b], t1 = cu[b + 1];
    if (!(0 <= t0 && t0 < t1 && t1 <= T) || !cu_ordered(cu, B)) return SeqInfo{0, 0, 0, 0};
    return SeqInfo{(size_t)t0, t1 - t0, t0 / kC + b, (t1 - t0 + kC - 1) / kC};
}

// Packed sequences: the sequence whose slot range may hold slot gc, the last b
// in [0, B) with floor(cu[b] / 64) + b <= gc (those bases increase with b).  A
// 64-way search, one wave: every lane tests one candidate per round, so B <= 64
// takes one round of loads and B <= 4096 two.  The result is wave-uniform.
__device__ __forceinline__ int find_seq(const int *cu, int B, int gc, int lane) {
    int lo = 0, n = B;  // the answer lies in [lo, lo + n)
    while (n > 1) {
        const int step = (n + 63) >> 6;
        const int cand = lo + lane * step;
        const bool le = lane * step < n && cu[cand] / kC + cand <= gc;
        const unsigned long long m = __ballot(le);
        const int j = m ? 63 - __clzll(m) : 0;
        lo += j * step;
        n = min(step, n - j * step);
    }
    return lo;
}

// e^x from the hardware base-2 exponential (v_exp_f32, about 1 ulp): the prep kernel is bound
// by VALU issue, and the library exp's range handling costs several instructions per call.
// Its arguments are log-decay sums (never positive past rounding); results that would be
// denormal flush to zero, which the decays they stand for are to fp16 precision anyway.
__device__ __forceinline__ float hw_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
// v when d >= 0, else +0, on the bit pattern: a select with an exponential in one arm is
// turned into a branch around it, and per element that costs more than the exponential.
// Where d < 0 the discarded v may be inf or NaN (an exponential of a positive argument).
__device__ __forceinline__ float keep_if_nonneg(int d, float v) {
    return __uint_as_float(__float_as_uint(v) & ~(unsigned int)(d >> 31));
}

__device__ __forceinline__ unsigned long long spin_load(unsigned long long *p, uint32_t tag, unsigned int *err,
                                                        int &broken) {
    // Wait until the tagged word at p carries `tag`.  Bounded: on a timeout the
    // error word is raised and this thread stops waiting for the rest of the
    // launch, so a lost sibling cannot stall every later chunk.
    unsigned long long w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t n = 0;
    while ((uint32_t)(w >> 32) != tag) {
        if (broken || ++n > kSpinLimit) {
            if (!broken) atomicOr(err, 1u);
            broken = 1;
            return 0ull;
        }
        __builtin_amdgcn_s_sleep(1);
        w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return w;
}

template <int N>
__device__ __forceinline__ int modn(int x) { return ((x % N) + N) % N; }

} // namespace
} // namespace gdn
