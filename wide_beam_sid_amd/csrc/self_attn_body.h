// Paged short-prefix self-attention over each beam row's own blocks: the
// device body shared by the self-attention kernel and the kernel that runs
// cross- and self-attention of a decode step in one launch.
//
// GRACE Section 5.2 (each beam row attends only to its own cached prefix:
// the block-diagonal mask, not a causal one, and the fused kernel that
// consumes q/k/v, writes the current token's k, v into the cache, gathers the
// prefix and returns the output) and Section 5.3 / Section 3.3 (flat KV pool
// of one-token blocks addressed through the block table P).
#pragma once

#include <cmath>
#include <type_traits>

#include "gr_device.h"
#include "gr_internal.h"

namespace gr {
namespace {

struct SelfParams {
    const void *q, *k_new, *v_new;
    void *k_pool, *v_pool;
    int32_t *table;
    void *out;
    int64_t fresh_base, pool_blocks;
    int R, t, L, H, d, E, G, CB;
    float scale_log2;   // log2(e) / sqrt(d_h)
};

// CB-byte pieces of a row: 4 or 8 bf16, 2 or 4 fp32.
template <bool BF16, int CB>
struct Chunk;
template <>
struct Chunk<true, 8> {
    static constexpr int VEC = 4;
    using W = uint2;
    __device__ static W zero() { return make_uint2(0u, 0u); }
    __device__ static void unpack(W u, float *f) {
        f[0] = __uint_as_float(u.x << 16);
        f[1] = __uint_as_float(u.x & 0xFFFF0000u);
        f[2] = __uint_as_float(u.y << 16);
        f[3] = __uint_as_float(u.y & 0xFFFF0000u);
    }
    __device__ static W pack(const float *f) {
        return make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
    }
};
template <>
struct Chunk<false, 8> {
    static constexpr int VEC = 2;
    using W = uint2;
    __device__ static W zero() { return make_uint2(0u, 0u); }
    __device__ static void unpack(W u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
    }
    __device__ static W pack(const float *f) {
        return make_uint2(__float_as_uint(f[0]), __float_as_uint(f[1]));
    }
};
template <>
struct Chunk<true, 16> {
    static constexpr int VEC = 8;
    using W = uint4;
    __device__ static W zero() { return make_uint4(0u, 0u, 0u, 0u); }
    __device__ static void unpack(W u, float *f) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[2 * e] = __uint_as_float(w[e] << 16);
            f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
    }
    __device__ static W pack(const float *f) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};
template <>
struct Chunk<false, 16> {
    static constexpr int VEC = 4;
    using W = uint4;
    __device__ static W zero() { return make_uint4(0u, 0u, 0u, 0u); }
    __device__ static void unpack(W u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ static W pack(const float *f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
};

// Beam rows of one workgroup (256 threads): LPR lanes per row, so 64 / LPR
// rows per wavefront.
template <int LPR>
constexpr int self_rows_wg() {
    return 4 * (64 / LPR);
}

// Sum over each aligned group of GC lanes (GC a power of two known at
// compile time): DPP steps within a 16-lane row (lane ^ 1, lane ^ 2, then
// the mirror image within 8 and 16 lanes, each pairing the two halves of a
// group), permutes across rows.
template <int GC>
__device__ __forceinline__ float group_sum_c(float v) {
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x),
                                                          decltype(ctrl)::value, 0xF, 0xF, false));
    };
    if constexpr (GC > 1) v += dpp(v, std::integral_constant<int, 0xB1>{});
    if constexpr (GC > 2) v += dpp(v, std::integral_constant<int, 0x4E>{});
    if constexpr (GC > 4) v += dpp(v, std::integral_constant<int, 0x141>{});
    if constexpr (GC > 8) v += dpp(v, std::integral_constant<int, 0x140>{});
    if constexpr (GC > 16) v += __shfl_xor(v, 16, 64);
    if constexpr (GC > 32) v += __shfl_xor(v, 32, 64);
    return v;
}

// Rows blk * self_rows_wg<LPR>() onwards.  A row's H*d_h elements are spread
// over LPR lanes in CB-byte pieces, NCH pieces per lane (NCH > 1 only with
// LPR = 64), so every load and store of a row is one coalesced access.  GC:
// the lanes of one head when known at compile time (0: p.G at run time).
template <bool BF16, int CB, int LPR, int NCH, int GC = 0>
__device__ __forceinline__ void self_attn_rows(const SelfParams &p, int blk) {
    using C = Chunk<BF16, CB>;
    using W = typename C::W;
    constexpr int VEC = C::VEC;
    constexpr int JB = NCH <= 2 ? 4 : (NCH <= 4 ? 2 : 1);   // prefix blocks per load batch
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lr = lane & (LPR - 1);
    const int i = blk * self_rows_wg<LPR>() + wave * (64 / LPR) + lane / LPR;
    if (i >= p.R) return;   // whole rows leave together
    const int E2 = p.E / VEC;  // pieces per row
    const int64_t f = p.fresh_base + i;
    const W *q = (const W *)p.q + (size_t)i * E2;
    const W *kn = (const W *)p.k_new + (size_t)i * E2;
    const W *vn = (const W *)p.v_new + (size_t)i * E2;
    W *kp = (W *)p.k_pool;
    W *vp = (W *)p.v_pool;

    // The first batch's block ids go out before the row's own loads and
    // the stores of its k, v: the gathers then wait for one round trip, not
    // two.
    // (Every lane loads every id of the batch, clamped to the row, and
    // drops those at or past t, so the loads are not behind branches.)
    int32_t bid0[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
        const int32_t v = p.table[(size_t)i * p.L + min(jj, p.L - 1)];
        bid0[jj] = jj < p.t ? v : -1;
    }

    // The row's q, k, v (a lane past the row's pieces reads its last one;
    // see the gathers below).  The current token's k, v and block id are
    // stored at the end: no position of this step reads block f, and a
    // store here would hold up the gathers' wait.
    float qf[NCH][VEC], kc[NCH][VEC], vc[NCH][VEC];
    float o[NCH][VEC], mrun[NCH], lrun[NCH];
    bool act[NCH];
    W ukp[NCH], uvp[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = c * LPR + lr;
        act[c] = e < E2;
        const int ec = min(e, E2 - 1);
        W uq = q[ec];
        ukp[c] = kn[ec];
        uvp[c] = vn[ec];
        if (!act[c]) uq = C::zero();
        C::unpack(uq, qf[c]);
        C::unpack(ukp[c], kc[c]);
        C::unpack(uvp[c], vc[c]);
        mrun[c] = -INFINITY;
        lrun[c] = 0.0f;
#pragma unroll
        for (int x = 0; x < VEC; ++x) o[c][x] = 0.0f;
    }

    // Prefix positions in batches of JB: the batch's block ids (one load,
    // the same address for the row's lanes), then every block load of the
    // batch before the first dot product; position t is the current token.
    for (int j0 = 0; j0 <= p.t; j0 += JB) {
        int32_t bid[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + jj;
            bid[jj] = j0 == 0 ? bid0[jj] : (j < p.t ? p.table[(size_t)i * p.L + j] : -1);
        }
        // Every lane loads a piece for every position of the batch, so the
        // loads are not behind branches and all of them are in flight
        // together: a position that is not used (past t, or a dead row's
        // missing past, skipped below) re-reads the lane's own q piece,
        // which the cache still holds, and a lane past the row's pieces
        // reads its last piece (its lanes form whole heads of their own,
        // whose results are never stored).
        W kr[JB][NCH], vr[JB][NCH];
        bool use[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + jj;
            // a dead row's missing past is skipped
            use[jj] = j < p.t && bid[jj] >= 0 && bid[jj] < p.pool_blocks;
            const W *ks = use[jj] ? kp + (size_t)bid[jj] * E2 : q;
            const W *vs = use[jj] ? vp + (size_t)bid[jj] * E2 : q;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int e = min(c * LPR + lr, E2 - 1);
                kr[jj][c] = ks[e];
                vr[jj][c] = vs[e];
            }
        }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + jj;
            if (j > p.t) break;                    // uniform
            const bool skip = j < p.t && !use[jj];   // the same for a row's lanes
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                float kj[VEC], vj[VEC];
                if (j < p.t) {
                    C::unpack(kr[jj][c], kj);
                    C::unpack(vr[jj][c], vj);
                } else {
#pragma unroll
                    for (int x = 0; x < VEC; ++x) {
                        kj[x] = kc[c][x];
                        vj[x] = vc[c][x];
                    }
                }
                float dot = 0.0f;
#pragma unroll
                for (int x = 0; x < VEC; ++x) dot += qf[c][x] * kj[x];
                // the G lanes of a head sit in one aligned group of the row
                if constexpr (GC > 0) {
                    dot = group_sum_c<GC>(dot);
                } else {
                    for (int o2 = p.G >> 1; o2 > 0; o2 >>= 1) dot += __shfl_xor(dot, o2, 64);
                }
                if (skip) continue;
                // The running max is taken over the raw dot products (the
                // scale is positive) and the scale applied after the
                // subtraction, which cannot contract into an FMA: the
                // maximal position's weight is exp2(0) = 1 exactly, so one
                // position returns its value unchanged.
                const float mn = fmaxf(mrun[c], dot);
                const float alpha = __builtin_amdgcn_exp2f((mrun[c] - mn) * p.scale_log2);
                const float pe = __builtin_amdgcn_exp2f((dot - mn) * p.scale_log2);
                lrun[c] = lrun[c] * alpha + pe;
#pragma unroll
                for (int x = 0; x < VEC; ++x) o[c][x] = o[c][x] * alpha + pe * vj[x];
                mrun[c] = mn;
            }
        }
    }
    W *out = (W *)p.out + (size_t)i * E2;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = c * LPR + lr;
        if (!act[c]) continue;
        kp[(size_t)f * E2 + e] = ukp[c];   // current token -> fresh block
        vp[(size_t)f * E2 + e] = uvp[c];
        const float inv = 1.0f / lrun[c];
        float r[VEC];
#pragma unroll
        for (int x = 0; x < VEC; ++x) r[x] = o[c][x] * inv;
        out[e] = C::pack(r);
    }
    if (lr == 0) p.table[(size_t)i * p.L + p.t] = (int32_t)f;
}

inline SelfParams self_params(const void *q, const void *k_new, const void *v_new, void *k_pool,
                              void *v_pool, int64_t pool_blocks, int32_t *table,
                              int64_t fresh_base, int R, int t, int L, int H, int d, gr_dtype dt,
                              void *out) {
    SelfParams p{};
    p.pool_blocks = pool_blocks;
    p.q = q;
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_pool = k_pool;
    p.v_pool = v_pool;
    p.table = table;
    p.out = out;
    p.fresh_base = fresh_base;
    p.R = R;
    p.t = t;
    p.L = L;
    p.H = H;
    p.d = d;
    p.E = H * d;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
    // 16-byte pieces when a head fills whole ones, else 8-byte pieces
    const int es = dt == GR_BF16 ? 2 : 4;
    p.CB = (d * es) % 16 == 0 ? 16 : 8;
    p.G = d * es / p.CB;   // lanes holding one head
    return p;
}

// Lanes per row (16, 32 or 64) and pieces per lane of the layout above.
struct SelfLayout {
    int lpr, nch;
};
inline SelfLayout self_layout(const SelfParams &p, bool bf16) {
    const int vec = p.CB / (bf16 ? 2 : 4);
    const int e2 = p.E / vec;
    if (p.CB == 16 && e2 <= 16) return {16, 1};
    if (p.CB == 16 && e2 <= 32) return {32, 1};
    return {64, (e2 + 63) / 64};
}

}  // namespace
}  // namespace gr
