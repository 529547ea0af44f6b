// Drives the host side of the loss library: every entry point of
// include/rl_post_loss.h with arguments that its validation must reject, at
// the edges of the shape limits (where an unguarded product of two int64
// sizes would overflow), and with valid arguments on a machine with no GPU
// (which must return RLPL_ERR_DEVICE and enqueue nothing); and the host
// helpers the launches are planned with (the exact row divisor, the split of
// logit rows) over wide argument ranges, checked against their definitions.
// Built host-only with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py, linked with the library's sources: any
// out-of-bounds access or undefined arithmetic aborts the run.  Prints
// "ok <checks>" and exits 0 when every check held.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <limits>

#include "rl_post_loss.h"
#include "row_divisor.h"
#include "vocab_kernels.h"

namespace {

long checks = 0, failures = 0;

void expect(bool ok, const char* what, long long a = 0, long long b = 0) {
    ++checks;
    if (!ok) {
        ++failures;
        fprintf(stderr, "FAIL %s (%lld, %lld)\n", what, a, b);
    }
}

uint64_t state = 0x2545f4914f6cdd1dull;
uint64_t next_u64() {   // splitmix64
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// Host stand-ins for device buffers: validation looks at addresses only.
alignas(256) unsigned char arena[1 << 22];
void* at(size_t off) { return arena + off; }

constexpr int64_t kBig = std::numeric_limits<int64_t>::max();
constexpr int64_t kMin = std::numeric_limits<int64_t>::min();
const int64_t kShapes[][2] = {{0, 1}, {1, 0}, {-1, 5}, {5, -1}, {kBig, kBig}, {kBig, 2}, {2, kBig},
                              {kMin, -1}, {-1, kMin}, {int64_t(1) << 31, 1}, {1, int64_t(1) << 31},
                              {int64_t(1) << 16, int64_t(1) << 15}, {int64_t(1) << 32, int64_t(1) << 32}};

int policy(int op, const void* lp, const void* old, const void* ref, const void* adv, const void* mask,
           int64_t bs, int64_t T, int dtype, int mdt, float beta, float eps, float eps_high, float* loss,
           void* grad, uint32_t* n, void* ws, size_t wsb) {
    return rlpl_policy_loss(op, 0, lp, old, ref, adv, mask, bs, T, dtype, mdt, beta, eps, eps_high, loss, grad, n,
                            ws, wsb, nullptr);
}

void policy_losses() {
    const size_t wsb = rlpl_workspace_bytes(64, 4096, RLPL_OP_BNPO);
    expect(wsb > 0 && wsb <= sizeof(arena) / 2, "workspace size");
    void* ws = at(sizeof(arena) / 2);
    float* loss = static_cast<float*>(at(4096));
    uint32_t* n = reinterpret_cast<uint32_t*>(at(4352));
    const void *lp = at(0), *old = at(512), *ref = at(1024), *adv = at(1536), *mask = at(2048);
    void* grad = at(2560);
    for (int op = -2; op < 6; ++op) {
        const bool policy_op = op >= 0 && op <= 3;
        const bool fused = op == 0 || op == 2;
        // A valid call: no device here.
        int st = policy(op, lp, old, ref, adv, mask, 64, 4096, RLPL_BF16, RLPL_MASK_INT8, 0.04f, 0.2f, 0.28f,
                        loss, grad, n, ws, wsb);
        expect(st == (policy_op ? RLPL_ERR_DEVICE : RLPL_ERR_PARAM), "valid call without a device", op, st);
        if (!policy_op) continue;
        for (const auto& s : kShapes) {
            st = policy(op, lp, old, ref, adv, mask, s[0], s[1], RLPL_BF16, RLPL_MASK_INT8, 0.04f, 0.2f, 0.28f,
                        loss, grad, n, ws, wsb);
            expect(st == RLPL_ERR_SHAPE, "shape", s[0], s[1]);
        }
        // Largest accepted shape: bs * seq_len = 2^31 - 1.
        st = policy(op, lp, old, ref, adv, mask, 1, (int64_t(1) << 31) - 1, RLPL_BF16, RLPL_MASK_INT8, 0.04f,
                    0.2f, 0.28f, loss, grad, n, ws, wsb);
        expect(st == RLPL_ERR_DEVICE, "largest shape", op, st);
        const struct { const char* what; int want; int st; } cases[] = {
            {"null mask", RLPL_ERR_NULL, policy(op, lp, old, ref, adv, nullptr, 4, 8, RLPL_F32, 0, 0.1f, 0.2f,
                                                0.2f, loss, grad, n, ws, wsb)},
            {"null loss", RLPL_ERR_NULL, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f, 0.2f, 0.2f,
                                                nullptr, grad, n, ws, wsb)},
            {"null policy", RLPL_ERR_NULL, policy(op, nullptr, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                  0.2f, 0.2f, loss, grad, n, ws, wsb)},
            {"null ref with beta", RLPL_ERR_NULL, policy(op, lp, old, nullptr, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                         0.2f, 0.2f, loss, grad, n, ws, wsb)},
            {"null ref without beta", RLPL_ERR_DEVICE, policy(op, lp, old, nullptr, adv, mask, 4, 8, RLPL_F32, 0,
                                                              0.0f, 0.2f, 0.2f, loss, grad, n, ws, wsb)},
            {"null grad", fused ? RLPL_ERR_NULL : RLPL_ERR_DEVICE,
             policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f, 0.2f, 0.2f, loss, nullptr, n, ws, wsb)},
            {"dtype", RLPL_ERR_DTYPE, policy(op, lp, old, ref, adv, mask, 4, 8, 3, 0, 0.1f, 0.2f, 0.2f, loss,
                                             grad, n, ws, wsb)},
            {"mask dtype", RLPL_ERR_DTYPE, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 2, 0.1f, 0.2f,
                                                  0.2f, loss, grad, n, ws, wsb)},
            {"plane alignment", RLPL_ERR_ALIGN, policy(op, at(8), old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                       0.2f, 0.2f, loss, grad, n, ws, wsb)},
            {"advantage alignment", RLPL_ERR_ALIGN, policy(op, lp, old, ref, at(1538), mask, 4, 8, RLPL_F32, 0,
                                                           0.1f, 0.2f, 0.2f, loss, grad, n, ws, wsb)},
            {"mask alignment", RLPL_ERR_ALIGN, policy(op, lp, old, ref, adv, at(2049), 4, 8, RLPL_F32, 0, 0.1f,
                                                      0.2f, 0.2f, loss, grad, n, ws, wsb)},
            {"count alignment", RLPL_ERR_ALIGN, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                       0.2f, 0.2f, loss, grad,
                                                       reinterpret_cast<uint32_t*>(at(4354)), ws, wsb)},
            {"workspace size", RLPL_ERR_WORKSPACE, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                          0.2f, 0.2f, loss, grad, n, ws, 1024)},
            {"null workspace", RLPL_ERR_WORKSPACE, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                          0.2f, 0.2f, loss, grad, n, nullptr, wsb)},
            {"workspace alignment", RLPL_ERR_ALIGN, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                           0.2f, 0.2f, loss, grad, n, at(sizeof(arena) / 2 - 128),
                                                           wsb)},
            {"nan beta", RLPL_ERR_PARAM, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, nanf(""), 0.2f,
                                                0.2f, loss, grad, n, ws, wsb)},
            {"infinite epsilon", RLPL_ERR_PARAM, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                        INFINITY, 0.2f, loss, grad, n, ws, wsb)},
            {"empty clip range", RLPL_ERR_PARAM, policy(op, lp, old, ref, adv, mask, 4, 8, RLPL_F32, 0, 0.1f,
                                                        0.5f, -0.7f, loss, grad, n, ws, wsb)},
        };
        for (const auto& c : cases) expect(c.st == c.want, c.what, op, c.st);
    }
    // The named entry points route to the same validation.
    expect(bnpo_loss(lp, old, ref, adv, nullptr, 4, 8, RLPL_BF16, 0, 0.f, 0.2f, 0.2f, loss, grad, n, ws, wsb,
                     nullptr) == RLPL_ERR_NULL, "bnpo_loss");
    expect(bnpo_loss_fwd(lp, old, ref, adv, mask, kBig, kBig, RLPL_BF16, 0, 0.f, 0.2f, 0.2f, loss, n, ws, wsb,
                         nullptr) == RLPL_ERR_SHAPE, "bnpo_loss_fwd");
    expect(grpo_loss(lp, old, ref, adv, mask, 4, 8, 7, 0, 0.f, 0.2f, 0.2f, loss, grad, n, ws, wsb, nullptr) ==
               RLPL_ERR_DTYPE, "grpo_loss");
    expect(grpo_loss_fwd(lp, old, ref, adv, mask, 4, 8, RLPL_F16, 0, 0.f, 0.2f, 0.2f, loss, n, ws, wsb, nullptr) ==
               RLPL_ERR_DEVICE, "grpo_loss_fwd");
    // The entry point without a workspace validates before it touches any device state.
    expect(bnpo_loss_noalloc(lp, old, ref, adv, mask, 64, 4096, RLPL_BF16, 1, 0.f, 0.2f, 0.28f, loss, grad, n,
                             nullptr) == RLPL_ERR_DEVICE, "noalloc valid");
    expect(bnpo_loss_noalloc(lp, old, ref, adv, mask, kBig, 3, RLPL_BF16, 1, 0.f, 0.2f, 0.28f, loss, grad, n,
                             nullptr) == RLPL_ERR_SHAPE, "noalloc shape");
    expect(bnpo_loss_noalloc(lp, old, ref, adv, mask, 64, 4096, RLPL_BF16, 1, 0.f, 0.2f, 0.28f, loss, nullptr, n,
                             nullptr) == RLPL_ERR_NULL, "noalloc grad");
}

void reverse_kl_losses() {
    const size_t wsb = rlpl_workspace_bytes(256, 8192, RLPL_OP_RKL);
    void* ws = at(sizeof(arena) / 2);
    float* loss = static_cast<float*>(at(4096));
    uint32_t* n = reinterpret_cast<uint32_t*>(at(4352));
    const void *s = at(0), *t = at(512), *mask = at(2048);
    void* grad = at(2560);
    expect(reverse_kl(s, t, mask, 256, 8192, RLPL_BF16, 0, loss, grad, n, ws, wsb, nullptr) == RLPL_ERR_DEVICE,
           "reverse_kl valid");
    expect(reverse_kl_fwd(s, t, mask, 256, 8192, RLPL_BF16, 0, loss, n, ws, wsb, nullptr) == RLPL_ERR_DEVICE,
           "reverse_kl_fwd valid");
    for (const auto& sh : kShapes) {
        expect(reverse_kl(s, t, mask, sh[0], sh[1], RLPL_BF16, 0, loss, grad, n, ws, wsb, nullptr) ==
                   RLPL_ERR_SHAPE, "reverse_kl shape", sh[0], sh[1]);
        expect(reverse_kl_fwd(s, t, mask, sh[0], sh[1], RLPL_BF16, 0, loss, n, ws, wsb, nullptr) == RLPL_ERR_SHAPE,
               "reverse_kl_fwd shape", sh[0], sh[1]);
    }
    expect(reverse_kl(nullptr, t, mask, 4, 8, RLPL_BF16, 0, loss, grad, n, ws, wsb, nullptr) == RLPL_ERR_NULL,
           "reverse_kl null");
    expect(reverse_kl(s, t, mask, 4, 8, RLPL_BF16, 0, loss, nullptr, n, ws, wsb, nullptr) == RLPL_ERR_NULL,
           "reverse_kl null grad");
    expect(reverse_kl(s, at(520), mask, 4, 8, RLPL_BF16, 0, loss, grad, n, ws, wsb, nullptr) == RLPL_ERR_ALIGN,
           "reverse_kl align");

    // Logit slabs: rows < 2^31 and rows * vocab <= 2^62.
    const size_t vwsb = rlpl_workspace_bytes(8, 248320, RLPL_OP_RKL_LOGITS);
    expect(vwsb > 0 && vwsb <= sizeof(arena) / 2, "vocab workspace size");
    expect(reverse_kl_logits(s, t, mask, 8, 248320, RLPL_BF16, 0, loss, grad, n, ws, vwsb, nullptr) ==
               RLPL_ERR_DEVICE, "reverse_kl_logits valid");
    expect(reverse_kl_logits_fwd(s, t, mask, 1, int64_t(1) << 62, RLPL_F32, 0, loss, n, ws, vwsb, nullptr) ==
               RLPL_ERR_DEVICE, "reverse_kl_logits_fwd largest vocab");
    const int64_t vshapes[][2] = {{0, 5}, {5, 0}, {-3, 7}, {int64_t(1) << 31, 1}, {2, (int64_t(1) << 61) + 1},
                                  {kBig, kBig}, {kMin, kMin}, {3, kBig}};
    for (const auto& sh : vshapes) {
        expect(reverse_kl_logits(s, t, mask, sh[0], sh[1], RLPL_BF16, 0, loss, grad, n, ws, vwsb, nullptr) ==
                   RLPL_ERR_SHAPE, "reverse_kl_logits shape", sh[0], sh[1]);
        expect(reverse_kl_logits_fwd(s, t, mask, sh[0], sh[1], RLPL_BF16, 0, loss, n, ws, vwsb, nullptr) ==
                   RLPL_ERR_SHAPE, "reverse_kl_logits_fwd shape", sh[0], sh[1]);
    }
    expect(reverse_kl_logits(s, t, mask, 8, 1000, RLPL_BF16, 0, loss, grad, n, ws, 4096, nullptr) ==
               RLPL_ERR_WORKSPACE, "reverse_kl_logits workspace");
    expect(reverse_kl_logits(s, t, at(2050), 8, 1000, RLPL_BF16, 0, loss, grad, n, ws, vwsb, nullptr) ==
               RLPL_ERR_ALIGN, "reverse_kl_logits mask align");
}

void logprob() {
    const int64_t shapes[][3] = {{0, 64, 64}, {4, 0, 64}, {4, 64, 0}, {-1, 64, 64}, {kBig, kBig, kBig},
                                 {4, kBig, 8}, {int64_t(1) << 40, 8, int64_t(1) << 40}};
    for (const auto& sh : shapes) {
        for (int back = 0; back < 2; ++back) {
            const size_t b = selective_logprob_workspace_bytes(sh[0], sh[1], sh[2], back);
            expect(b == 0, "logprob workspace of a rejected shape", sh[0], sh[1]);
        }
        expect(selective_logprob_fwd(at(0), at(1024), nullptr, static_cast<const int64_t*>(at(2048)), sh[0], sh[1],
                                     sh[2], RLPL_BF16, static_cast<float*>(at(4096)), nullptr,
                                     at(sizeof(arena) / 2), sizeof(arena) / 2, nullptr) == RLPL_ERR_SHAPE,
               "logprob shape", sh[0], sh[2]);
    }
    const int64_t N = 1024, H = 4096, V = 32000;
    const size_t fb = selective_logprob_workspace_bytes(N, H, V, 0);
    const size_t bb = selective_logprob_workspace_bytes(N, H, V, 1);
    expect(fb > 0 && bb >= fb, "logprob workspace sizes");
    const int64_t* tg = static_cast<const int64_t*>(at(2048));
    float* lp = static_cast<float*>(at(4096));
    // The workspace is never dereferenced on the host, so any aligned address serves.
    void* ws = reinterpret_cast<void*>(uintptr_t(1) << 40);
    expect(selective_logprob_fwd(at(0), at(1024), nullptr, tg, N, H, V, RLPL_BF16, lp, nullptr, ws, fb,
                                 nullptr) == RLPL_ERR_DEVICE, "logprob fwd valid");
    expect(selective_logprob_fwd(at(0), at(1024), nullptr, tg, N, H, V, RLPL_F32, lp, nullptr, ws, fb, nullptr) ==
               RLPL_ERR_DTYPE, "logprob dtype");
    expect(selective_logprob_fwd(at(0), at(1024), nullptr, tg, N, H, V, RLPL_BF16, lp, nullptr, ws, fb - 1,
                                 nullptr) == RLPL_ERR_WORKSPACE, "logprob workspace");
    expect(selective_logprob_bwd(at(0), at(1024), nullptr, tg, lp, lp, N, H, V, RLPL_BF16, at(8192),
                                 static_cast<float*>(at(16384)), nullptr, 0, ws, bb, nullptr) == RLPL_ERR_DEVICE,
           "logprob bwd valid");
    expect(selective_logprob_bwd(at(0), at(1024), nullptr, tg, lp, lp, N, H, V, RLPL_BF16, at(8192),
                                 static_cast<float*>(at(16384)), nullptr, 0, ws, fb - 1, nullptr) ==
               RLPL_ERR_WORKSPACE, "logprob bwd workspace");
}

void queries() {
    for (int op = -3; op < 12; ++op)
        for (const auto& s : kShapes) (void)rlpl_workspace_bytes(s[0], s[1], op);
    expect(rlpl_workspace_bytes(4, 8, 99) == 0, "workspace bytes of a bad op");
    for (int st = -4; st < 16; ++st) expect(rlpl_status_string(st) != nullptr, "status string", st);
    expect(rlpl_version() >= 1, "version");
    int g = -1, v = -1, t = -1;
    expect(rlpl_launch_shape(64, 4096, RLPL_BF16, RLPL_OP_BNPO, &g, &v, &t) == RLPL_ERR_DEVICE, "launch shape");
    expect(rlpl_launch_shape(kBig, kBig, RLPL_BF16, RLPL_OP_BNPO, &g, &v, &t) == RLPL_ERR_SHAPE,
           "launch shape of a bad shape");
    expect(rlpl_launch_shape(64, 4096, RLPL_BF16, RLPL_OP_BNPO, nullptr, &v, &t) == RLPL_ERR_NULL,
           "launch shape null");
    uint32_t flags = 0;
    expect(rlpl_workspace_flags(nullptr, &flags, nullptr) != RLPL_OK, "flags of a null workspace");
    expect(rlpl_workspace_flags(at(256), nullptr, nullptr) != RLPL_OK, "flags into a null pointer");
    expect(rlpl_workspace_set_limits(nullptr, 1, 1, 1, nullptr) != RLPL_OK, "limits of a null workspace");
    expect(rlpl_workspace_set_limits(at(8), 1, 1, 1, nullptr) == RLPL_ERR_ALIGN, "limits alignment");
}

void row_divisors() {
    for (int i = 0; i < 4000; ++i) {
        uint32_t d;
        switch (i % 4) {
        case 0: d = 1 + uint32_t(next_u64() % 4096); break;
        case 1: d = 1 + uint32_t(next_u64() % 0x7FFFFFFFu); break;
        case 2: d = uint32_t(1) << (next_u64() % 31); break;
        default: d = (uint32_t(1) << (1 + next_u64() % 30)) - 1; break;
        }
        uint32_t magic = 0, shift = 0;
        const bool ok = rlpl::row_divisor(d, &magic, &shift);
        expect(ok, "row divisor exists", d);
        if (!ok) continue;
        for (int k = 0; k < 64; ++k) {
            const uint32_t n = k < 8 ? uint32_t(0x7FFFFFFFu - k) : uint32_t(next_u64() & 0x7FFFFFFFu);
            const uint32_t q = uint32_t((uint64_t(n) * magic) >> shift);
            if (q != n / d) expect(false, "row divisor quotient", d, n);
        }
    }
    uint32_t m = 0, s = 0;
    expect(!rlpl::row_divisor(0, &m, &s) && !rlpl::row_divisor(0x80000000u, &m, &s), "row divisor domain");
}

void vocab_splits() {
    for (int i = 0; i < 20000; ++i) {
        const int64_t rows = 1 + int64_t(next_u64() % (i % 3 == 0 ? 4 : (i % 3 == 1 ? 5000 : 2000000)));
        const int64_t vocab = 1 + int64_t(next_u64() % (i % 2 ? 300000 : 8000000));
        const int elem = (i % 3 == 0) ? 4 : 2;
        const int64_t cap = 1 + int64_t(next_u64() % 4096);
        const bool fused = next_u64() & 1;
        const rlpl::VocabSplit sp = rlpl::vocab_split(rows, vocab, elem, cap, fused);
        const int64_t per_block = 32 / elem;
        const int64_t blocks = vocab % per_block == 0 ? vocab / per_block : vocab / per_block + 2;
        const bool ok = sp.chunks >= 1 && sp.chunks <= rlpl::kVocabMaxChunks && sp.chunk_blocks >= 1 &&
                        sp.chunks * sp.chunk_blocks >= blocks && (sp.chunks - 1) * sp.chunk_blocks < blocks &&
                        sp.groups >= 0 && sp.groups <= rows && sp.groups * sp.chunks <= (cap > sp.chunks ? cap : sp.chunks);
        if (!ok) expect(false, "vocab split", rows, vocab);
        ++checks;
    }
}

}  // namespace

int main() {
    policy_losses();
    reverse_kl_losses();
    logprob();
    queries();
    row_divisors();
    vocab_splits();
    printf("ok %ld\n", checks);
    return failures ? 1 : 0;
}
