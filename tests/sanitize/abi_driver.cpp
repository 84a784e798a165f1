// Host-side argument checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_sanitizers.py).  Every
// call below is rejected by a host check before any HIP call, so it needs no GPU
// and never touches the buffers it is given: host arrays stand in for device
// memory, and are sized so that any read or write through them would be caught.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gdn.h"

static int failures = 0;
#define EXPECT_EQ(a, b)                                                                                  \
    do {                                                                                                 \
        const long long va = (long long)(a), vb = (long long)(b);                                        \
        if (va != vb) {                                                                                  \
            std::fprintf(stderr, "FAIL line %d: %s = %lld, expected %lld\n", __LINE__, #a, va, vb);      \
            ++failures;                                                                                  \
        }                                                                                                \
    } while (0)

static gdn_shape make(int B, int T, int Hk, int Hv) {
    gdn_shape s;
    std::memset(&s, 0, sizeof s);
    s.B = B; s.T = T; s.Hk = Hk; s.Hv = Hv; s.Dk = 128; s.Dv = 128; s.conv_width = 4;
    s.eps_l2 = 1e-6f; s.eps_norm = 1e-6f;
    return s;
}

// 16-byte aligned, non-overlapping stand-ins for the device buffers of a small shape
struct Bufs {
    std::vector<unsigned char> mem;
    unsigned char *base;
    size_t used = 0;
    explicit Bufs(size_t bytes) : mem(bytes + 64) {
        base = mem.data() + (16 - (reinterpret_cast<uintptr_t>(mem.data()) & 15)) % 16;
    }
    template <class T> T *take(size_t bytes) {
        T *p = reinterpret_cast<T *>(base + used);
        used += (bytes + 255) / 256 * 256;
        return p;
    }
};

int main() {
    // status strings, including codes the library never returns
    for (int st = 2; st >= -9; --st)
        if (!gdn_status_string(st) || !*gdn_status_string(st)) ++failures;
    if (!gdn_last_error()) ++failures;

    // ---- shapes
    size_t ws = 0;
    gdn_shape s = make(1, 256, 1, 2);
    EXPECT_EQ(gdn_prefill_workspace_size(&s, &ws), GDN_OK);
    if (ws == 0) ++failures;
    EXPECT_EQ(gdn_prefill_workspace_size(nullptr, &ws), GDN_EINVAL);
    EXPECT_EQ(gdn_prefill_workspace_size(&s, nullptr), GDN_EINVAL);
    gdn_shape b = s; b.Dk = 64;             EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EUNSUPPORTED);
    b = s; b.conv_width = 3;                EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EUNSUPPORTED);
    b = s; b.Hv = 3;                        EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_OK);
    b = s; b.Hk = 2; b.Hv = 3;              EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.T = 0;                         EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.B = -1;                        EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.flags = 8;                     EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.eps_l2 = -1.0f;                EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.eps_norm = 0.0f / 0.0f;        EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.prefill_segments = -1;         EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.flags = GDN_PACKED; b.prefill_segments = 2; EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.prefill_segments = 1000000;    EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_OK);  // capped
    b = s; b.T = 0x7fffffff;                EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);
    b = s; b.B = 0x40000000; b.Hv = 64; b.Hk = 64; EXPECT_EQ(gdn_prefill_workspace_size(&b, &ws), GDN_EINVAL);

    // ---- prefill buffers of shape s (B=1, T=256, Hk=1, Hv=2)
    EXPECT_EQ(gdn_prefill_workspace_size(&s, &ws), GDN_OK);
    const size_t rows = 256, Cc = 2 * 128 + 2 * 128;
    const size_t nqk = rows * 128 * 2, nv = rows * 2 * 128 * 2, ngb = rows * 2 * 4, nst = 2 * 128 * 128 * 4;
    Bufs m(8 * nqk + 4 * nv + 4 * ngb + 3 * nst + 8 * Cc * 8 + ws + (1 << 16));
    auto *q = m.take<uint16_t>(nqk), *k = m.take<uint16_t>(nqk), *v = m.take<uint16_t>(nv), *z = m.take<uint16_t>(nv);
    auto *g = m.take<float>(ngb), *beta = m.take<float>(ngb);
    auto *conv_w = m.take<uint16_t>(Cc * 8), *norm_w = m.take<uint16_t>(256);
    auto *o = m.take<uint16_t>(nv);
    auto *state_out = m.take<float>(nst);
    auto *cs_out = m.take<uint16_t>(3 * Cc * 2);
    void *work = m.take<void>(ws);
    auto call = [&](const gdn_shape &sh, const uint16_t *qq, const uint16_t *oo, void *wk, size_t wb) {
        return gdn_prefill(&sh, qq, k, v, g, beta, z, conv_w, norm_w, nullptr, nullptr, const_cast<uint16_t *>(oo),
                           state_out, cs_out, wk, wb, nullptr);
    };
    EXPECT_EQ(call(s, nullptr, o, work, ws), GDN_EINVAL);                                  // null q
    EXPECT_EQ(call(s, q + 1, o, work, ws), GDN_EINVAL);                                    // misaligned q
    EXPECT_EQ(call(s, q, q, work, ws), GDN_EINVAL);                                        // o overlaps q
    EXPECT_EQ(call(s, q, o, work, ws - 1), GDN_EWORKSPACE);                                // workspace short by 1 B
    EXPECT_EQ(call(s, q, o, reinterpret_cast<unsigned char *>(o) + 16, ws), GDN_EINVAL);   // workspace over o
    EXPECT_EQ(gdn_prefill(&s, q, k, v, g, beta, z, nullptr, norm_w, nullptr, nullptr, o, state_out, cs_out, work, ws,
                          nullptr), GDN_EINVAL);                                           // conv without weights
    EXPECT_EQ(gdn_prefill(&s, q, k, v, g, beta, nullptr, conv_w, norm_w, nullptr, nullptr, o, state_out, cs_out, work,
                          ws, nullptr), GDN_EINVAL);                                       // norm without z
    EXPECT_EQ(gdn_prefill(&s, q, k, v, reinterpret_cast<const float *>(reinterpret_cast<const char *>(g) + 2), beta,
                          z, conv_w, norm_w, nullptr, nullptr, o, state_out, cs_out, work, ws, nullptr),
              GDN_EINVAL);                                                                 // g not 4-byte aligned
    EXPECT_EQ(gdn_prefill(&s, q, k, v, g, beta, z, conv_w, norm_w, state_out + 1, nullptr, o, state_out, cs_out, work,
                          ws, nullptr), GDN_EINVAL);                                       // state in/out partly overlap
    gdn_shape sp = s; sp.flags = GDN_PACKED;
    EXPECT_EQ(call(sp, q, o, work, ws), GDN_EINVAL);                                       // packed without cu_seqlens
    int32_t cu[2] = {0, 256};
    EXPECT_EQ(gdn_prefill_packed(&s, cu, q, k, v, g, beta, z, conv_w, norm_w, nullptr, nullptr, o, state_out, cs_out,
                                 work, ws, nullptr), GDN_EINVAL);                          // cu_seqlens on an even batch
    EXPECT_EQ(gdn_prefill_gate_logits(&s, q, k, v, g, beta, nullptr, nullptr, z, conv_w, norm_w, nullptr, nullptr, o,
                                      state_out, cs_out, work, ws, nullptr), GDN_EINVAL);  // gate logits without A_log
    gdn_shape s0 = s; s0.conv_width = 0;
    EXPECT_EQ(gdn_prefill(&s0, q, k, v, g, beta, z, nullptr, norm_w, nullptr, nullptr, o, state_out, cs_out, work, ws,
                          nullptr), GDN_EINVAL);                                           // conv tail without conv
    EXPECT_EQ(gdn_prefill_check(nullptr, 4096, nullptr), GDN_EINVAL);
    EXPECT_EQ(gdn_prefill_check(work, 16, nullptr), GDN_EINVAL);
    EXPECT_EQ(gdn_prefill_check(static_cast<unsigned char *>(work) + 4, ws, nullptr), GDN_EINVAL);

    // ---- decode
    gdn_shape d = make(2, 1, 1, 2);
    auto *state = m.take<float>(2 * nst);
    auto *cs = m.take<uint16_t>(2 * 3 * Cc * 2);
    EXPECT_EQ(gdn_decode_step(&d, q, k, v, g, beta, z, conv_w, norm_w, state, nullptr, o, nullptr), GDN_EINVAL);
    EXPECT_EQ(gdn_decode_step(&d, q, k, v, g, beta, z, conv_w, norm_w, nullptr, cs, o, nullptr), GDN_EINVAL);
    gdn_shape dm = d; dm.T = 9;
    EXPECT_EQ(gdn_decode_multi(&dm, q, k, v, g, beta, z, conv_w, norm_w, state, cs, o, nullptr, nullptr, nullptr),
              GDN_EINVAL);
    dm.T = 0;
    EXPECT_EQ(gdn_decode_multi(&dm, q, k, v, g, beta, z, conv_w, norm_w, state, cs, o, nullptr, nullptr, nullptr),
              GDN_EINVAL);
    gdn_shape dp = d; dp.flags = GDN_PACKED;
    EXPECT_EQ(gdn_decode_step(&dp, q, k, v, g, beta, z, conv_w, norm_w, state, cs, o, nullptr), GDN_EINVAL);
    EXPECT_EQ(gdn_decode_step(&d, q, k, v, g, beta, z, conv_w, norm_w, state, cs, reinterpret_cast<uint16_t *>(state),
                              nullptr), GDN_EINVAL);                                       // o overlaps the state
    EXPECT_EQ(gdn_state_init(nullptr, state, cs, nullptr), GDN_EINVAL);
    EXPECT_EQ(gdn_state_init(&d, state + 1, cs, nullptr), GDN_EINVAL);
    gdn_shape dn = d; dn.conv_width = 0;
    EXPECT_EQ(gdn_state_init(&dn, state, cs, nullptr), GDN_EINVAL);

    if (failures) std::fprintf(stderr, "%d check(s) failed\n", failures);
    else std::printf("abi host checks: all passed\n");
    return failures ? 1 : 0;
}
