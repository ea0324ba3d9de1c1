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
    int R, t, L, H, d, E, G;
    float scale;
};

template <bool BF16>
struct Chunk;
template <>
struct Chunk<true> {  // 4 x bf16 in 8 bytes
    static constexpr int VEC = 4;
    __device__ static void unpack(uint2 u, float *f) {
        f[0] = __uint_as_float(u.x << 16);
        f[1] = __uint_as_float(u.x & 0xFFFF0000u);
        f[2] = __uint_as_float(u.y << 16);
        f[3] = __uint_as_float(u.y & 0xFFFF0000u);
    }
    __device__ static uint2 pack(const float *f) {
        return make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
    }
};
template <>
struct Chunk<false> {  // 2 x fp32 in 8 bytes
    static constexpr int VEC = 2;
    __device__ static void unpack(uint2 u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
    }
    __device__ static uint2 pack(const float *f) {
        return make_uint2(__float_as_uint(f[0]), __float_as_uint(f[1]));
    }
};

// Rows blk * 4 .. blk * 4 + 3, one per wavefront of a 256-thread workgroup.
template <bool BF16, int NCH>
__device__ __forceinline__ void self_attn_rows(const SelfParams &p, int blk) {
    using C = Chunk<BF16>;
    constexpr int VEC = C::VEC;
    constexpr int JB = NCH <= 2 ? 4 : (NCH <= 4 ? 2 : 1);   // prefix blocks per load batch
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = blk * 4 + wave;
    if (i >= p.R) return;
    const int E2 = p.E / VEC;  // 8-byte chunks per row
    const int64_t f = p.fresh_base + i;
    const uint2 *q = (const uint2 *)p.q + (size_t)i * E2;
    const uint2 *kn = (const uint2 *)p.k_new + (size_t)i * E2;
    const uint2 *vn = (const uint2 *)p.v_new + (size_t)i * E2;
    uint2 *kp = (uint2 *)p.k_pool;
    uint2 *vp = (uint2 *)p.v_pool;

    float qf[NCH][VEC], kc[NCH][VEC], vc[NCH][VEC];
    float o[NCH][VEC], mrun[NCH], lrun[NCH];
    bool act[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = c * 64 + lane;
        act[c] = e < E2;
        uint2 uq = make_uint2(0, 0), uk = uq, uv = uq;
        if (act[c]) {
            uq = q[e];
            uk = kn[e];
            uv = vn[e];
            kp[(size_t)f * E2 + e] = uk;   // current token -> fresh block
            vp[(size_t)f * E2 + e] = uv;
        }
        C::unpack(uq, qf[c]);
        C::unpack(uk, kc[c]);
        C::unpack(uv, vc[c]);
        mrun[c] = -INFINITY;
        lrun[c] = 0.0f;
#pragma unroll
        for (int x = 0; x < VEC; ++x) o[c][x] = 0.0f;
    }
    // The row's prefix block ids, lane j holding position j (L <= 64).
    const int32_t tb = lane < p.t ? p.table[(size_t)i * p.L + lane] : -1;
    if (lane == 0) p.table[(size_t)i * p.L + p.t] = (int32_t)f;

    // Prefix positions in batches of JB: every block load of a batch is
    // issued before the first dot product, then the current token.
    for (int j0 = 0; j0 <= p.t; j0 += JB) {
        uint2 kr[JB][NCH], vr[JB][NCH];
        bool use[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + jj;
            const int32_t blk = __builtin_amdgcn_readlane(tb, j < 64 ? j : 0);
            // a dead row's missing past is skipped; position t is the current token
            use[jj] = j < p.t && blk >= 0 && blk < p.pool_blocks;
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int e = c * 64 + lane;
                kr[jj][c] = vr[jj][c] = make_uint2(0, 0);
                if (use[jj] && act[c]) {
                    kr[jj][c] = kp[(size_t)blk * E2 + e];
                    vr[jj][c] = vp[(size_t)blk * E2 + e];
                }
            }
        }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + jj;
            if (j > p.t) break;                  // uniform
            if (j < p.t && !use[jj]) continue;   // uniform
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
                for (int o2 = p.G >> 1; o2 > 0; o2 >>= 1) dot += __shfl_xor(dot, o2, 64);
                const float sc = dot * p.scale;
                const float mn = fmaxf(mrun[c], sc);
                const float alpha = __expf(mrun[c] - mn);
                const float pe = __expf(sc - mn);
                lrun[c] = lrun[c] * alpha + pe;
#pragma unroll
                for (int x = 0; x < VEC; ++x) o[c][x] = o[c][x] * alpha + pe * vj[x];
                mrun[c] = mn;
            }
        }
    }
    uint2 *out = (uint2 *)p.out + (size_t)i * E2;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int e = c * 64 + lane;
        if (!act[c]) continue;
        const float inv = 1.0f / lrun[c];
        float r[VEC];
#pragma unroll
        for (int x = 0; x < VEC; ++x) r[x] = o[c][x] * inv;
        out[e] = C::pack(r);
    }
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
    p.scale = 1.0f / sqrtf((float)d);
    p.G = dt == GR_BF16 ? d / 4 : d / 2;   // lanes holding one head
    return p;
}

// 8-byte chunks of a row (4 bf16 or 2 fp32) per lane, in multiples of 64.
inline int self_chunks(const SelfParams &p, bool bf16) {
    return (p.E / (bf16 ? 4 : 2) + 63) / 64;
}

}  // namespace
}  // namespace gr
