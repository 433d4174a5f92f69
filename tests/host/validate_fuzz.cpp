// Randomised checks of the host-side argument checker (gemv_validate.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitize.py.  Every entry point is called with random
// arguments: extreme and negative sizes, null, unaligned, overlapping and
// wrapping pointers, malformed views.  For each call it checks that the
// status is a documented one, that a second identical call returns the same
// status (the checker keeps no state), and, where gemv_validate or
// gemv_fused_ncols_validate accepts a call, that dst truly overlaps neither W
// nor x and meets its operand only as the identical view, with byte spans
// computed here in 128-bit integers, and that none of its buffers runs past
// the top of the address space.  Exits 1 on the first violation; the
// sanitizers abort on any undefined behaviour or bad memory access.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "gemv_fused.h"

namespace {

typedef unsigned __int128 u128;

struct Rng {
    uint64_t s;
    uint64_t next()
    {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
    bool coin(int pct) { return (int64_t)(next() % 100) < pct; }
};

// A size: mostly small, sometimes at or beyond the documented limits.
int64_t pick_size(Rng &r)
{
    static const int64_t edge[] = {0, -1, 1, 31, 32, 33, 64, 1024, 4096, 14336,
                                   (1LL << 31) - 1, 1LL << 31, (1LL << 31) + 1, 1LL << 40, INT64_MAX, INT64_MIN};
    if (r.coin(20))
        return edge[r.next() % (sizeof(edge) / sizeof(edge[0]))];
    return r.coin(50) ? 32 * r.range(1, 8) : r.range(1, 300);
}

// Addresses from a small pool so that buffers overlap often, plus a few that
// are null, unaligned or near the top of the address space.
uintptr_t pick_addr(Rng &r)
{
    if (r.coin(3))
        return 0;
    if (r.coin(3))
        return UINTPTR_MAX - (uintptr_t)r.range(0, 4096);
    uintptr_t a = 0x100000 + 256 * (uintptr_t)r.range(0, 64);
    if (r.coin(10))
        a += (uintptr_t)r.range(1, 15);
    return a;
}

void pick_view(Rng &r, gemv_view &v, int64_t want_numel)
{
    v.data = reinterpret_cast<float *>(pick_addr(r));
    v.ndim = r.coin(5) ? (int32_t)r.range(-1, 6) : (int32_t)r.range(1, 4);
    int64_t n = want_numel > 0 && want_numel < (1LL << 31) && r.coin(80) ? want_numel : pick_size(r);
    for (int d = 0; d < GEMV_MAX_DIMS; ++d) {
        v.shape[d] = 1;
        v.stride[d] = 1;
    }
    const int nd = v.ndim >= 1 && v.ndim <= GEMV_MAX_DIMS ? v.ndim : 1;
    if (n > 0 && r.coin(50) && nd >= 2 && n % 32 == 0) {
        v.shape[nd - 2] = 32;
        v.shape[nd - 1] = n / 32;
    } else {
        v.shape[nd - 1] = n;
    }
    if (r.coin(5))
        v.shape[r.next() % nd] = pick_size(r);
    int64_t st = 1;
    for (int d = nd - 1; d >= 0; --d) {
        v.stride[d] = st;
        if (v.shape[d] > 0 && v.shape[d] < (1LL << 31) && st < (1LL << 31))
            st *= v.shape[d];
    }
    if (r.coin(5))
        v.stride[r.next() % nd] = pick_size(r);
}

bool valid_status(int s) { return s <= GEMV_OK && s >= GEMV_E_HIP; }

// Independent byte count of the weights, or -1 where the arguments are not valid.
__int128 weight_bytes_ref(int wfmt, int64_t N, int64_t K)
{
    if (wfmt < GEMV_W_F32 || wfmt > GEMV_W_Q4B32 || N < 1 || K < 1 || N >= (1LL << 31) || K >= (1LL << 31))
        return -1;
    const __int128 nk = (__int128)N * K;
    auto a256 = [](__int128 v) { return (v + 255) / 256 * 256; };
    switch (wfmt) {
    case GEMV_W_F32:
        return nk * 4;
    case GEMV_W_F16:
    case GEMV_W_BF16:
        return nk * 2;
    case GEMV_W_Q8B32:
        return K % 32 ? -1 : a256(nk) + (__int128)N * (K / 32) * 2;
    default:
        return K % 32 ? -1 : a256(nk / 2) + (__int128)N * (K / 32) * 2;
    }
}

bool disjoint(uintptr_t a, u128 abytes, uintptr_t b, u128 bbytes)
{
    const u128 alo = a, ahi = (u128)a + abytes, blo = b, bhi = (u128)b + bbytes;
    return ahi <= blo || bhi <= alo;
}

int failures = 0;
void fail(const char *what, long it)
{
    std::fprintf(stderr, "violation at iteration %ld: %s\n", it, what);
    if (++failures > 10)
        std::exit(1);
}

} // namespace

int main(int argc, char **argv)
{
    const long iters = argc > 1 ? std::atol(argv[1]) : 200000;
    Rng r{0x5EEDull};
    for (long it = 0; it < iters; ++it) {
        const int wfmt = (int)r.range(-1, 5);
        const int64_t N = pick_size(r), K = pick_size(r);
        const int act = (int)r.range(-1, 6);
        const void *W = reinterpret_cast<const void *>(pick_addr(r));
        const float *x = reinterpret_cast<const float *>(pick_addr(r));
        const int64_t ncols = r.coin(80) ? r.range(1, 8) : pick_size(r);

        const int64_t wb = gemv_weight_bytes(wfmt, N, K);
        const __int128 wref = weight_bytes_ref(wfmt, N, K);
        if (wb >= 0 && (__int128)wb != wref)
            fail("gemv_weight_bytes disagrees with the 128-bit count", it);
        if (wb < 0 && wref >= 0 && wref < ((__int128)1 << 62))
            fail("gemv_weight_bytes rejects a representable size", it);

        gemv_view dst, mul, add;
        const int64_t nout = ncols >= 1 && ncols <= 8 && N > 0 && N < (1LL << 31) ? N * ncols : N;
        pick_view(r, dst, nout);
        pick_view(r, mul, nout);
        pick_view(r, add, nout);
        if (r.coin(15))
            mul = dst;
        if (r.coin(15))
            add = dst;
        const gemv_view *mp = r.coin(50) ? &mul : nullptr;
        const gemv_view *ap = r.coin(50) ? &add : nullptr;
        const gemv_view *dp = r.coin(2) ? nullptr : &dst;

        // one column
        const int s1 = gemv_validate(W, wfmt, N, K, x, act, mp, ap, dp);
        if (!valid_status(s1) || s1 != gemv_validate(W, wfmt, N, K, x, act, mp, ap, dp))
            fail("gemv_validate status", it);
        // several columns
        const int sc = gemv_fused_ncols_validate(W, wfmt, N, K, ncols, x, act, mp, ap, dp);
        if (!valid_status(sc) || sc != gemv_fused_ncols_validate(W, wfmt, N, K, ncols, x, act, mp, ap, dp))
            fail("gemv_fused_ncols_validate status", it);
        if (sc == GEMV_OK) {
            const u128 db = (u128)N * ncols * 4;
            const uintptr_t d = reinterpret_cast<uintptr_t>(dp->data);
            if (wref < 0 || !disjoint(d, db, (uintptr_t)W, (u128)wref))
                fail("accepted dst overlapping W", it);
            if (!disjoint(d, db, (uintptr_t)x, (u128)ncols * K * 4))
                fail("accepted dst overlapping x", it);
            const gemv_view *op = act == GEMV_ACT_ADD ? ap : ((act == GEMV_ACT_MUL || act == GEMV_ACT_SILU_MUL) ? mp : nullptr);
            if (op && op->data != dp->data && !disjoint(d, db, reinterpret_cast<uintptr_t>(op->data), db))
                fail("accepted a partial overlap of dst and the operand", it);
            if (reinterpret_cast<uintptr_t>(W) % 16 || reinterpret_cast<uintptr_t>(x) % 4 || d % 4)
                fail("accepted a misaligned pointer", it);
            const u128 top = (u128)1 << 64;
            if ((u128)(uintptr_t)W + (u128)wref > top || (u128)(uintptr_t)x + (u128)ncols * K * 4 > top ||
                (u128)d + db > top || (op && (u128)reinterpret_cast<uintptr_t>(op->data) + db > top))
                fail("accepted a buffer that runs past the top of the address space", it);
        }
        if (ncols == 1 && s1 != sc)
            fail("gemv_validate and the one-column ncols check disagree", it);

        // gated pair, epilogue pass, Hadamard transform, transform + product
        const void *W2 = reinterpret_cast<const void *>(pick_addr(r));
        const int sg = gemv_glu_validate(W, W2, wfmt, N, K, x, act, dp);
        if (!valid_status(sg) || sg != gemv_glu_validate(W, W2, wfmt, N, K, x, act, dp))
            fail("gemv_glu_validate status", it);
        const int sgn = gemv_glu_ncols_validate(W, W2, wfmt, N, K, ncols, x, act, dp);
        if (!valid_status(sgn) || sgn != gemv_glu_ncols_validate(W, W2, wfmt, N, K, ncols, x, act, dp))
            fail("gemv_glu_ncols_validate status", it);
        if (ncols == 1 && sgn != sg)
            fail("gemv_glu_ncols_validate with one column and gemv_glu_validate disagree", it);
        if (sgn == GEMV_OK) {
            const u128 db = (u128)N * ncols * 4;
            const uintptr_t d = reinterpret_cast<uintptr_t>(dp->data);
            if (wref < 0 || !disjoint(d, db, (uintptr_t)W, (u128)wref) || !disjoint(d, db, (uintptr_t)W2, (u128)wref) ||
                !disjoint(d, db, (uintptr_t)x, (u128)ncols * K * 4))
                fail("gemv_glu_ncols_validate accepted dst overlapping a matrix or x", it);
        }
        const int se = gemv_epilogue_validate(act, N, x, mp, ap, dp);
        if (!valid_status(se) || se != gemv_epilogue_validate(act, N, x, mp, ap, dp))
            fail("gemv_epilogue_validate status", it);
        const int64_t n = r.coin(70) ? (1LL << r.range(0, 11)) : pick_size(r);
        const int64_t nsigns = r.coin(70) ? K : pick_size(r);
        const int64_t nrows = r.coin(70) ? r.range(1, 8) : pick_size(r);
        const float *signs = reinterpret_cast<const float *>(pick_addr(r));
        float *fdst = reinterpret_cast<float *>(pick_addr(r));
        const int sf = gemv_fwht_signed_validate(x, signs, nrows, K, n, nsigns, fdst);
        if (!valid_status(sf) || sf != gemv_fwht_signed_validate(x, signs, nrows, K, n, nsigns, fdst))
            fail("gemv_fwht_signed_validate status", it);
        const int sp = gemv_fused_fwht_validate(W, wfmt, N, K, x, signs, n, nsigns, act, mp, ap, dp);
        if (!valid_status(sp) || sp != gemv_fused_fwht_validate(W, wfmt, N, K, x, signs, n, nsigns, act, mp, ap, dp))
            fail("gemv_fused_fwht_validate status", it);
        for (int s : {s1, sc, sg, sgn, se, sf, sp})
            if (!gemv_strerror(s))
                fail("gemv_strerror returned NULL", it);
    }
    if (failures)
        return 1;
    std::printf("ok %ld iterations\n", iters);
    return 0;
}
