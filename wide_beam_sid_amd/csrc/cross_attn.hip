// Beam-as-query cross-attention on gfx950.
//
// GRACE Section 5.1, eqs 11-14 and Appendix B: the context K, V stay at
// request granularity [B, H, T_ctx, d_h] and the M beam rows of a request are
// that request's query sequence, so one K/V tile load serves every beam of the
// request.  The flattening is request-major (row b*M + m), which is the
// layout bijection of eqs 13-14: no data moves, only the indexing changes.
//
// bf16 path: one workgroup = one (request, head) and 64 or 128 beam rows
// (4 wavefronts x 1 or 2 blocks of 16 rows).  Per 64-key tile (double
// buffered), K is staged in LDS row-major and V transposed; S^T = K Q^T and
// O^T += V^T P^T run on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation and an online softmax in
// registers.  Computing the transposed products keeps each lane on one query
// row: its S values are exactly the B operand of the P.V product (the
// key order inside a 32-wide k step is permuted identically for V), and its
// output is a contiguous run of d for one row, stored as 16-byte writes.
// fp32 path (small heads): one wavefront per (row, head), lanes over d.
#include "gr_device.h"
#include "gr_internal.h"
#include "self_attn_body.h"

namespace gr {
namespace {

constexpr int TT = 64;          // keys per LDS tile
constexpr int PAD = 8;          // bf16 padding per LDS row
constexpr int BUF_DWORD3 = 0x00020000;   // buffer descriptor word 3 for gfx9 raw loads

union V8 {
    uint4 u;
    bf16x8 b;
};

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Two fp32 values to a bf16 pair (round to nearest even), low half first.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{lo, hi}, bf16x2v));
}

// The beam-prefix part of the joint attention: the current token's k, v
// (written to block fresh_base + r) and the row's earlier blocks P[r, j < t].
struct JointArgs {
    const uint16_t *k_new, *v_new;
    uint16_t *k_pool, *v_pool;
    int32_t *table;
    int64_t pool_blocks, fresh_base;
    int t, L;
};

// Split-K: the workgroup covers keys [k0, k1) only and leaves, for split s,
// its unnormalised output (fp32) and the row's running max (scaled log2
// units) and normaliser in po / pml, which k_cross_merge combines.
struct SplitArgs {
    int k0, k1, s, R;
    float *po;    // [S, R, H, D]
    float *pml;   // [S, R, H, 2]
};

// One workgroup = (request b, head h, 64 * RB beam rows); wavefront w takes
// RB blocks of 16 rows.  The K / V tiles of 64 keys are double-buffered in
// LDS: the global loads of tile i + 1 are in flight (in registers) while
// tile i is computed, then written to the other buffer, one barrier per
// tile.  K is stored row-major; V transposed, two keys per 32-bit store,
// each row's dword columns XOR-swizzled so the P.V reads are free of bank
// conflicts.
//
// JOINT: after the context tiles, the same online softmax continues over the
// row's own beam positions j = 0..t (shared-prefix beam attention): lane
// (g, a) dots its quarter of row a's query with the position's key, the four
// lanes of the row sum their parts, and the lane's output columns take the
// weighted value; position t is the current token, which also goes to the
// pool.  One output, no partial results leave the kernel.
template <int D, int RB, bool JOINT, bool RAG, bool SPLIT = false, int NBUF = 2>
__device__ __forceinline__ void cross_rows(const uint16_t *__restrict__ q,
                                           const uint16_t *__restrict__ K,
                                           const uint16_t *__restrict__ Vv,
                                           uint16_t *__restrict__ out, int M, int H, int T,
                                           float scale_log2, const JointArgs &jn, int bx, int h,
                                           int b, const SplitArgs &sp = SplitArgs{}) {
    const int k0 = SPLIT ? sp.k0 : 0, k1 = SPLIT ? sp.k1 : T;   // keys of this workgroup
    constexpr int NDC = D / 32;   // k steps of S = Q K^T
    constexpr int NDB = D / 16;   // 16-wide blocks of d in O^T
    constexpr int ROWS = 4 * RB * 16;
    constexpr int KIT = TT * (D / 8);              // 16-byte K pieces per tile
    constexpr int VIT = (TT / 2) * (D / 8);        // (key pair, 8 d) V pieces per tile
    constexpr int KU = (KIT + 255) / 256, VU = (VIT + 255) / 256;
    // NBUF = 2: double-buffered tiles.  NBUF = 1 (the standalone d_h = 128
    // kernel): one buffer, 33 KB of LDS instead of 66 KB, so three
    // workgroups fit a CU instead of two; the next tile's loads are still in
    // flight (in registers) over the current tile's products, and one more
    // barrier per tile guards the buffer before they are stored.
    static_assert(NBUF == 1 || NBUF == 2, "tile buffers");
    __shared__ __attribute__((aligned(16))) uint16_t sK[NBUF][TT][D + PAD];
    // V^T as key pairs, row d of TT / 2 dwords, the dword column XORed with
    // vsw(d), so the 16 rows a 16-lane pass of the P.V product reads (d & 3
    // and d / (D / 4) varying) fall on distinct banks (padded rows instead
    // leave 4-way conflicts: rows d and d + 16 of a 36-dword pitch share a
    // bank; the joint kernel at two row blocks ran 2-3% faster swizzled).
    constexpr int VP = TT / 2;   // dwords per V^T row
    __shared__ __attribute__((aligned(16))) uint32_t sVt[NBUF][D][VP];
    static_assert(D == 32 || D == 64 || D == 128, "head size");
    constexpr int SHV = D == 32 ? 3 : (D == 64 ? 4 : 5);   // log2(D / 4)
    auto vsw = [](int d) { return 2 * ((d & 3) | (((d >> SHV) & 3) << 2)); };

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, a = lane & 15;
    // every row d this lane reads in the P.V product has vsw(d) = 2a, so
    // its four V^T dword columns are vc0 ^ {0, 8, 16, 24}
    const int vc0 = (2 * g) ^ (2 * a);
    const int mbase = bx * ROWS + wave * RB * 16;
    const size_t kvbase = ((size_t)b * H + h) * (size_t)T * D;

    // K / V tiles through buffer loads: the (request, head) slice is the
    // buffer (T * D bf16), each lane's offset inside a tile is fixed and the
    // tile's start goes in the scalar offset.  Keys past T fall outside the
    // buffer and read as zeros, so a ragged last tile needs no branches.
    const uint32_t nbytes = (uint32_t)T * D * 2;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void *)(K + kvbase), (short)0, nbytes, BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void *)(Vv + kvbase), (short)0, nbytes, BUF_DWORD3);
    uint32_t ko[KU], vo[VU];
#pragma unroll
    for (int u = 0; u < KU; ++u) {
        const int it = tid + u * 256, key = it / (D / 8), dc = it % (D / 8);
        ko[u] = (uint32_t)(key * D + dc * 8) * 2;
    }
#pragma unroll
    for (int u = 0; u < VU; ++u) {
        // consecutive threads take consecutive key pairs of one 8-wide d
        // block, so the transposed stores below fill consecutive dwords
        const int it = tid + u * 256, dc = it / (TT / 2), kp = it % (TT / 2);
        vo[u] = (uint32_t)(2 * kp * D + dc * 8) * 2;
    }
    auto ld16 = [](__amdgpu_buffer_rsrc_t r, uint32_t vo, uint32_t so) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0);
        return make_uint4(x[0], x[1], x[2], x[3]);
    };
    uint4 kr[KU], vr[VU][2];
    auto load_tile = [&](int t0) {
        const uint32_t so = (uint32_t)t0 * D * 2;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            kr[u] = make_uint4(0u, 0u, 0u, 0u);
            if (KIT % 256 == 0 || tid + u * 256 < KIT) kr[u] = ld16(rk, ko[u], so);
        }
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            vr[u][0] = vr[u][1] = make_uint4(0u, 0u, 0u, 0u);
            if (VIT % 256 == 0 || tid + u * 256 < VIT) {
                vr[u][0] = ld16(rv, vo[u], so);
                vr[u][1] = ld16(rv, vo[u] + D * 2, so);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int u = 0; u < KU; ++u) {
            const int it = tid + u * 256, key = it / (D / 8), dc = it % (D / 8);
            if (it < KIT) *(uint4 *)&sK[buf][key][dc * 8] = kr[u];
        }
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            const int it = tid + u * 256, dc = it / (TT / 2), kp = it % (TT / 2);
            if (it < VIT) {
                const uint32_t w0[4] = {vr[u][0].x, vr[u][0].y, vr[u][0].z, vr[u][0].w};
                const uint32_t w1[4] = {vr[u][1].x, vr[u][1].y, vr[u][1].z, vr[u][1].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r0 = dc * 8 + 2 * e, r1 = r0 + 1;
                    sVt[buf][r0][kp ^ vsw(r0)] = (w0[e] & 0xFFFFu) | (w1[e] << 16);
                    sVt[buf][r1][kp ^ vsw(r1)] = (w0[e] >> 16) | (w1[e] & 0xFFFF0000u);
                }
            }
        }
    };

    load_tile(k0);
    // Q^T as the B operand: lane (g, a) holds Q[row a][c*32 + g*8 .. +8];
    // these loads stay in flight over the first tile's LDS stores and
    // barrier.
    // The request's M rows are one buffer, so rows past M read as zeros
    // and every lane issues the same loads (no branch around them).
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(q + (size_t)b * M * H * D), (short)0, (uint32_t)M * H * D * 2, BUF_DWORD3);
    bf16x8 qf[RB][NDC];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = mbase + rb * 16 + a;
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            V8 t;
            t.u = ld16(rq, (uint32_t)(((size_t)m * H + h) * D + c * 32 + g * 8) * 2, 0);
            qf[rb][c] = t.b;
        }
    }
    f32x4 o[RB][NDB];
    // osum: the product of an all-ones V^T block with P^T, i.e. the row's
    // running normaliser (the sum of the weights the product uses), in every
    // element of each lane of the row
    f32x4 osum[RB];
    // VOTE (four row blocks per wavefront, where the vector work of the
    // tile bounds the kernel): the growth test on each lane's own maximum;
    // with fewer row blocks the test on the row's maximum measured faster.
    constexpr bool VOTE = RB >= 4;
    // thr: the raw dot product above which a row's weights would pass 2^8
    // (mrow + 8 in scaled log2 units; a rounding either way only moves a
    // rescale by a tile, and any running max gives the same output)
    float mrow[RB], lpart[RB], thr[RB];
    const float inv_scale = 1.0f / scale_log2;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        mrow[rb] = -INFINITY;
        thr[rb] = -INFINITY;
        lpart[rb] = 0.0f;
        osum[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    store_tile(0);
    __syncthreads();

    // One 64-key tile: the next tile's loads go out first, the products
    // and the softmax run on the current buffer, then the next tile is
    // stored to the other one.  The first tile is peeled off the loop and
    // waits for every load still in flight (the Q fragments) before it
    // issues the second tile's, so that neither it nor the loop, where the
    // only loads in flight are the next tile's, holds its products for
    // them.
    auto key_tile = [&](int t0, int cur, bool first) {
        const bool more = t0 + TT < k1;
        const int cb = NBUF == 1 ? 0 : cur;   // the buffer holding this tile
        if (first) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0) only
        if (more) load_tile(t0 + TT);
        // S^T block kb of row block rb: lane holds S[row a][key t0 + kb*16 +
        // g*4 + i].  Each K fragment read from LDS serves every row block.
        f32x4 s[RB][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) s[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int c = 0; c < NDC; ++c) {
                V8 ka;
                ka.u = *(const uint4 *)&sK[cb][kb * 16 + a][c * 32 + g * 8];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
                    s[rb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka.b, qf[rb][c], s[rb][kb], 0, 0, 0);
            }
        // The max runs over the raw dot products (the scale is positive); the
        // running max m is kept in scaled log2 units, and each weight is
        // exp2(s * scale_log2 - m) with the scale folded into one FMA.  Keys
        // past T exist only in a ragged last tile (RAG).
        float tm[RB];
        bool grow = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (RAG && t0 + kb * 16 + g * 4 + i >= T) s[rb][kb][i] = -INFINITY;
                    tmax = fmaxf(tmax, s[rb][kb][i]);
                }
            if constexpr (VOTE) {
                tm[rb] = tmax;   // this lane's part of the row (raw dot products)
                grow = grow || tmax > thr[rb];
            } else {
                tm[rb] = pair32_max(pair16_max(tmax)) * scale_log2;   // over the row's 4 lanes g
                grow = grow || tm[rb] > mrow[rb] + 8.0f;
            }
        }
        // The running maxima move only when a row's tile max exceeds its
        // running max by more than 8 (log2 units): the weights then stay
        // below 2^8, and the rescale of the outputs and normalisers is
        // skipped on most tiles (one uniform branch for the wavefront's row
        // blocks).  Any max gives the same normalised output.  VOTE: a row's
        // tile max exceeds the bound exactly when one of its four lanes'
        // maxima does, so the test votes on the lanes' own maxima and the
        // maxima over the row's lanes are taken only on the (rare) rescale.
        if (__ballot(grow)) {
            if constexpr (VOTE)
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)   // over the row's 4 lanes g
                    tm[rb] = pair32_max(pair16_max(tm[rb])) * scale_log2;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float mnew = fmaxf(mrow[rb], tm[rb]);
                thr[rb] = (mnew + 8.0f) * inv_scale;
                const float alpha = __builtin_amdgcn_exp2f(mrow[rb] - mnew);
                mrow[rb] = mnew;
                osum[rb] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[rb][db] *= alpha;
            }
        }
        uint32_t pk[RB][4][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float mcur = mrow[rb];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int hp = 0; hp < 2; ++hp)
                    pk[rb][kb][hp] = cvt_bf16x2(
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][kb][2 * hp], scale_log2, -mcur)),
                        __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][kb][2 * hp + 1], scale_log2, -mcur)));
        }
        // O^T += V^T P^T, k step over keys of sub-blocks (2pc, 2pc+1):
        // slot g*8+i <-> key (2pc)*16 + g*4 + i (i < 4),
        //                    (2pc+1)*16 + g*4 + i-4 (i >= 4).
        // Each V^T fragment read from LDS serves every row block.
#pragma unroll
        for (int pc = 0; pc < 2; ++pc) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                // A row a <-> d = (a/4)*4*NDB + db*4 + a%4
                const int d = (a >> 2) * (4 * NDB) + db * 4 + (a & 3);
                const uint2 lo = *(const uint2 *)&sVt[cb][d][vc0 ^ (pc * 16)];
                const uint2 hi = *(const uint2 *)&sVt[cb][d][vc0 ^ (pc * 16 + 8)];
                V8 va;
                va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    V8 pb;
                    pb.u = make_uint4(pk[rb][2 * pc][0], pk[rb][2 * pc][1], pk[rb][2 * pc + 1][0],
                                      pk[rb][2 * pc + 1][1]);
                    o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.b, pb.b, o[rb][db], 0, 0, 0);
                }
            }
            V8 ones;   // bf16 1.0 in every slot
            ones.u = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                V8 pb;
                pb.u = make_uint4(pk[rb][2 * pc][0], pk[rb][2 * pc][1], pk[rb][2 * pc + 1][0],
                                  pk[rb][2 * pc + 1][1]);
                osum[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones.b, pb.b, osum[rb], 0, 0, 0);
            }
        }
        if (more) {
            if (NBUF == 1) __syncthreads();   // every wavefront is done with the buffer
            store_tile(NBUF == 1 ? 0 : cur ^ 1);
        }
        __syncthreads();
    };
    key_tile(k0, 0, true);
    for (int t0 = k0 + TT, cur = 1; t0 < k1; t0 += TT, cur ^= 1) key_tile(t0, cur, false);
    // the normaliser as a partial per lane, summed over the row's 4 lanes below
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lpart[rb] = g == 0 ? osum[rb][0] : 0.0f;

    if constexpr (JOINT) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int m = mbase + rb * 16 + a;
            const bool rv = m < M;
            const size_t r = (size_t)b * M + (rv ? m : 0);
            const int64_t fblk = jn.fresh_base + (int64_t)r;
            for (int j = 0; j <= jn.t; ++j) {
                // position j < t: block P[r, j] (skipped when missing); j = t:
                // the current token
                int64_t blk = fblk;
                bool use = rv;
                if (j < jn.t) {
                    blk = rv ? jn.table[r * jn.L + j] : -1;
                    use = rv && blk >= 0 && blk < jn.pool_blocks;
                }
                const uint16_t *kr = j < jn.t ? jn.k_pool + ((size_t)(use ? blk : 0) * H + h) * D
                                              : jn.k_new + (r * H + h) * D;
                const uint16_t *vr = j < jn.t ? jn.v_pool + ((size_t)(use ? blk : 0) * H + h) * D
                                              : jn.v_new + (r * H + h) * D;
                uint4 kc[NDC], vc[NDB / 2];
#pragma unroll
                for (int c = 0; c < NDC; ++c)
                    kc[c] = use ? *(const uint4 *)(kr + c * 32 + g * 8) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int c = 0; c < NDB / 2; ++c)
                    vc[c] = use ? *(const uint4 *)(vr + g * 4 * NDB + c * 8) : make_uint4(0u, 0u, 0u, 0u);
                if (j == jn.t && rv) {   // the current token's k, v to its fresh block
#pragma unroll
                    for (int c = 0; c < NDC; ++c)
                        *(uint4 *)(jn.k_pool + ((size_t)fblk * H + h) * D + c * 32 + g * 8) = kc[c];
#pragma unroll
                    for (int c = 0; c < NDB / 2; ++c)
                        *(uint4 *)(jn.v_pool + ((size_t)fblk * H + h) * D + g * 4 * NDB + c * 8) = vc[c];
                    if (h == 0 && g == 0) jn.table[r * jn.L + jn.t] = (int32_t)fblk;
                }
                float dot = 0.0f;
#pragma unroll
                for (int c = 0; c < NDC; ++c) {
                    V8 kk;
                    kk.u = kc[c];
#pragma unroll
                    for (int e = 0; e < 8; ++e) dot += (float)qf[rb][c][e] * (float)kk.b[e];
                }
                dot = pair32_sum(pair16_sum(dot));
                const float sj = use ? dot * scale_log2 : -INFINITY;
                const float mn = fmaxf(mrow[rb], sj);
                const float al = __builtin_amdgcn_exp2f(mrow[rb] - mn);
                const float pj = __builtin_amdgcn_exp2f(sj - mn);
                mrow[rb] = mn;
                lpart[rb] = lpart[rb] * al + (g == 0 ? pj : 0.0f);   // counted once per row
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint32_t w0 = ((const uint32_t *)&vc[(db * 4) >> 3])[((db * 4) & 7) >> 1];
                    const uint32_t w1 = ((const uint32_t *)&vc[(db * 4) >> 3])[(((db * 4) & 7) >> 1) + 1];
                    const float vv[4] = {__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u),
                                         __uint_as_float(w1 << 16), __uint_as_float(w1 & 0xFFFF0000u)};
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[rb][db][i] = o[rb][db][i] * al + pj * vv[i];
                }
            }
        }
    }

    // Lane (g, a) holds O[row a][d = g*4*NDB + db*4 + i].
    if constexpr (SPLIT) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const float lt = pair32_sum(pair16_sum(lpart[rb]));
            const int m = mbase + rb * 16 + a;
            if (m >= M) continue;
            const size_t rh = ((size_t)sp.s * sp.R + (size_t)b * M + m) * H + h;
            float *dst = sp.po + rh * D + g * 4 * NDB;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                *(float4 *)(dst + db * 4) = make_float4(o[rb][db][0], o[rb][db][1], o[rb][db][2],
                                                        o[rb][db][3]);
            if (g == 0) *(float2 *)(sp.pml + rh * 2) = make_float2(mrow[rb], lt);
        }
        return;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float lt = lpart[rb];
        lt = pair32_sum(pair16_sum(lt));
        const float inv = 1.0f / lt;
        const int m = mbase + rb * 16 + a;
        if (m >= M) continue;
        uint32_t w[2 * NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            w[2 * db] = cvt_bf16x2(o[rb][db][0] * inv, o[rb][db][1] * inv);
            w[2 * db + 1] = cvt_bf16x2(o[rb][db][2] * inv, o[rb][db][3] * inv);
        }
        uint16_t *dst = out + (((size_t)b * M + m) * H + h) * D + g * 4 * NDB;
#pragma unroll
        for (int c = 0; c < NDB / 2; ++c)
            *(uint4 *)(dst + c * 8) = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
    }
}

// XCD-aware tile order.  The dispatcher hands workgroup w to XCD w mod 8,
// so workgroup w takes tile (w mod 8) * (n / 8) + w / 8: each XCD gets a
// contiguous run of tiles, and the row blocks of one (request, head), which
// are adjacent in the tile order, read their K / V through one L2 instead of
// eight.  Workgroups past the last multiple of 8 keep their own index.
__device__ __forceinline__ int xcd_tile(int w, int n) {
    const int per = n >> 3;
    return w < (per << 3) ? (w & 7) * per + (w >> 3) : w;
}

// One workgroup per (row block, head, request) tile; tiles are numbered
// row block fastest, then head, then request.
template <int D, int RB, bool JOINT, bool RAG>
__global__ __launch_bounds__(256, 2) void k_cross_bf16(const uint16_t *__restrict__ q,
                                                       const uint16_t *__restrict__ K,
                                                       const uint16_t *__restrict__ Vv,
                                                       uint16_t *__restrict__ out, int M, int H,
                                                       int T, float scale_log2, int gxc,
                                                       int n_tiles, JointArgs jn) {
    const int tile = xcd_tile(blockIdx.x, n_tiles);
    const int bx = tile % gxc, rest = tile / gxc;
    cross_rows<D, RB, JOINT, RAG, false, D == 128 ? 1 : 2>(q, K, Vv, out, M, H, T, scale_log2, jn,
                                                          bx, rest % H, rest / H);
}

// Split-K tiles: workgroup w takes tile-split x = xcd_tile(w, n) with the
// split fastest (tile = x / S, split s = x mod S); split s covers keys
// [s * Ts, min(T, (s + 1) * Ts)), Ts a multiple of the 64-key tile.  One
// row block per wavefront: the split path serves launches with few tiles.
template <int D, bool RAG>
__global__ __launch_bounds__(256, 2) void k_cross_split(const uint16_t *__restrict__ q,
                                                        const uint16_t *__restrict__ K,
                                                        const uint16_t *__restrict__ Vv, int M,
                                                        int H, int T, float scale_log2, int gxc,
                                                        int n, int S, int Ts, int R,
                                                        float *__restrict__ po,
                                                        float *__restrict__ pml) {
    const int x = xcd_tile(blockIdx.x, n);
    const int tile = x / S, s = x - tile * S;
    const int bx = tile % gxc, rest = tile / gxc;
    SplitArgs sp;
    sp.k0 = s * Ts;
    sp.k1 = min(T, sp.k0 + Ts);
    sp.s = s;
    sp.R = R;
    sp.po = po;
    sp.pml = pml;
    cross_rows<D, 1, false, RAG, true>(q, K, Vv, nullptr, M, H, T, scale_log2, JointArgs{}, bx,
                                       rest % H, rest / H, sp);
}

// The S splits of one (row, head) combined with a log-sum-exp: with
// c_s = 2^(m_s - max m), out = sum_s c_s o_s / sum_s c_s l_s, to bf16.
// One wavefront per (row, head), D / 64 elements per lane (at least one).
template <int D>
__global__ __launch_bounds__(256) void k_cross_merge(const float *__restrict__ po,
                                                     const float *__restrict__ pml,
                                                     uint16_t *__restrict__ out, int RH, int S) {
    constexpr int EPL = D >= 64 ? D / 64 : 1;
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (w >= RH) return;
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, pml[((size_t)s * RH + w) * 2]);
    float l = 0.0f, acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    for (int s = 0; s < S; ++s) {
        const float2 ml = *(const float2 *)(pml + ((size_t)s * RH + w) * 2);
        const float c = __builtin_amdgcn_exp2f(ml.x - mx);
        l += c * ml.y;
        const float *src = po + ((size_t)s * RH + w) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            if (lane * EPL + e < D) acc[e] += c * src[lane * EPL + e];
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
        if (lane * EPL + e < D) {
            const uint32_t pk = cvt_bf16x2(acc[e] * inv, 0.0f);
            out[(size_t)w * D + lane * EPL + e] = (uint16_t)(pk & 0xFFFFu);
        }
}

// Cross- and self-attention of one decode step in one launch (they are
// independent): the first n_cross workgroups take the cross-attention tiles
// (in the XCD-aware order above), the rest take the self-attention
// rows (4 to 16 per workgroup, by row width).  Saves a launch and lets the MFMA-bound tiles and the
// gather-bound rows share the machine.
template <int D, int RB, bool RAG, int LPR, int NCH>
__global__ __launch_bounds__(256, 2) void k_attn_pair(const uint16_t *__restrict__ q,
                                                      const uint16_t *__restrict__ K,
                                                      const uint16_t *__restrict__ Vv,
                                                      uint16_t *__restrict__ out, int M, int H,
                                                      int T, float scale_log2, int gxc,
                                                      int n_cross, SelfParams sp) {
    const int blk = blockIdx.x;
    if (blk < n_cross) {
        const int tile = xcd_tile(blk, n_cross);
        const int bx = tile % gxc, rest = tile / gxc;
        const JointArgs nj{};
        cross_rows<D, RB, false, RAG>(q, K, Vv, out, M, H, T, scale_log2, nj, bx, rest % H,
                                      rest / H);
    } else {
        self_attn_rows<true, 16, LPR, NCH, D / 8>(sp, blk - n_cross);   // a head: D * 2 / 16 lanes
    }
}

// fp32: one wavefront per (row, head), lane x holds q[x], online softmax.
__global__ __launch_bounds__(256) void k_cross_f32(const float *__restrict__ q,
                                                   const float *__restrict__ K,
                                                   const float *__restrict__ Vv,
                                                   float *__restrict__ out, int M, int H, int T,
                                                   int D, int rows, float scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int idx = blockIdx.x * 4 + wave;
    if (idx >= rows * H) return;
    const int r = idx / H, h = idx % H, b = r / M;
    const bool act = lane < D;
    const float qx = act ? q[((size_t)r * H + h) * D + lane] : 0.0f;
    const float *Kb = K + ((size_t)b * H + h) * (size_t)T * D;
    const float *Vb = Vv + ((size_t)b * H + h) * (size_t)T * D;
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    for (int tau = 0; tau < T; ++tau) {
        const float s = wave_sum(act ? qx * Kb[(size_t)tau * D + lane] : 0.0f) * scale;
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn);
        const float pe = expf(s - mn);
        l = l * alpha + pe;
        o = o * alpha + pe * (act ? Vb[(size_t)tau * D + lane] : 0.0f);
        m = mn;
    }
    if (act) out[((size_t)r * H + h) * D + lane] = o / l;
}

// fp32 joint attention: one wavefront per (row, head), lane x holds
// element x; the context keys, then the row's beam positions j = 0..t, in
// one online softmax.
__global__ __launch_bounds__(256) void k_joint_f32(const float *__restrict__ q,
                                                   const float *__restrict__ K,
                                                   const float *__restrict__ Vv,
                                                   const float *__restrict__ k_new,
                                                   const float *__restrict__ v_new, float *k_pool,
                                                   float *v_pool, int32_t *table,
                                                   int64_t pool_blocks, int64_t fresh_base,
                                                   float *__restrict__ out, int M, int H, int T,
                                                   int D, int rows, int t, int L, float scale) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int idx = blockIdx.x * 4 + wave;
    if (idx >= rows * H) return;
    const int r = idx / H, h = idx % H, b = r / M;
    const bool act = lane < D;
    const float qx = act ? q[((size_t)r * H + h) * D + lane] : 0.0f;
    const float *Kb = K + ((size_t)b * H + h) * (size_t)T * D;
    const float *Vb = Vv + ((size_t)b * H + h) * (size_t)T * D;
    float m = -INFINITY, l = 0.0f, o = 0.0f;
    auto push = [&](float s, float v) {
        const float mn = fmaxf(m, s);
        const float alpha = expf(m - mn);
        const float pe = expf(s - mn);
        l = l * alpha + pe;
        o = o * alpha + pe * v;
        m = mn;
    };
    for (int tau = 0; tau < T; ++tau)
        push(wave_sum(act ? qx * Kb[(size_t)tau * D + lane] : 0.0f) * scale,
             act ? Vb[(size_t)tau * D + lane] : 0.0f);
    const int64_t fblk = fresh_base + r;
    for (int j = 0; j < t; ++j) {
        const int64_t blk = table[(size_t)r * L + j];
        if (blk < 0 || blk >= pool_blocks) continue;   // a dead row's missing past
        const size_t o2 = ((size_t)blk * H + h) * D + lane;
        push(wave_sum(act ? qx * k_pool[o2] : 0.0f) * scale, act ? v_pool[o2] : 0.0f);
    }
    const float kx = act ? k_new[((size_t)r * H + h) * D + lane] : 0.0f;
    const float vx = act ? v_new[((size_t)r * H + h) * D + lane] : 0.0f;
    if (act) {
        k_pool[((size_t)fblk * H + h) * D + lane] = kx;
        v_pool[((size_t)fblk * H + h) * D + lane] = vx;
    }
    if (h == 0 && lane == 0) table[(size_t)r * L + t] = (int32_t)fblk;
    push(wave_sum(qx * kx) * scale, vx);
    if (act) out[((size_t)r * H + h) * D + lane] = o / l;
}

// The bf16 tile kernel for head size d, rb = 1, 2 or 4 row blocks per
// wavefront (4: d_h <= 64 only) and a ragged last key tile or none (rag).
template <bool JOINT>
hipError_t launch_cross_tiles(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                              uint16_t *out, int M, int H, int T, int d, float sl2, int gxc,
                              int n, int rb, bool rag, const JointArgs &jn, hipStream_t s) {
#define GR_TILES(DD, RBB, RG) \
    k_cross_bf16<DD, RBB, JOINT, RG><<<n, 256, 0, s>>>(q, k, v, out, M, H, T, sl2, gxc, n, jn)
#define GR_TILES_R(DD, RBB)        \
    {                              \
        if (rag) GR_TILES(DD, RBB, true); \
        else GR_TILES(DD, RBB, false);    \
    }
    if (d == 32) {
        if (rb == 4) GR_TILES_R(32, 4) else if (rb == 2) GR_TILES_R(32, 2) else GR_TILES_R(32, 1)
    } else if (d == 64) {
        if (rb == 4) GR_TILES_R(64, 4) else if (rb == 2) GR_TILES_R(64, 2) else GR_TILES_R(64, 1)
    } else {
        GR_TILES_R(128, 1)
    }
#undef GR_TILES_R
#undef GR_TILES
    return hipGetLastError();
}

}  // namespace

CrossSplit cross_split_plan(int B, int M, int H, int T, int d, gr_dtype dt) {
    CrossSplit p{1, T, 0};
    if (dt != GR_BF16 || (d != 32 && d != 64 && d != 128)) return p;
    const int64_t n_tiles = (int64_t)((M + 63) / 64) * H * B;   // one row block per wavefront
    const int nkt = (T + TT - 1) / TT;                           // 64-key tiles
    // two workgroups per CU fill the chip at 512 tiles; below that a long
    // key loop (8 tiles or more) is split so that about 1024 workgroups
    // run, each over at least four key tiles (shorter splits lost to the
    // extra merge launch: a 256-key context ran 1.5x slower split)
    if (n_tiles >= 512 || nkt < 8) return p;
    const int64_t want = (1024 + n_tiles - 1) / n_tiles;
    const int S0 = (int)(want < nkt / 4 ? want : nkt / 4);
    if (S0 < 2) return p;
    const int tps = (nkt + S0 - 1) / S0;
    const int Ts = tps * TT, S = (T + Ts - 1) / Ts;
    if (S < 2) return p;
    p.S = S;
    p.Ts = Ts;
    p.bytes = (size_t)S * B * M * H * (d + 2) * sizeof(float);
    return p;
}

hipError_t launch_cross_split(const void *q, const void *k, const void *v, void *out, int B,
                              int M, int H, int T, int d, const CrossSplit &pl, void *ws,
                              hipStream_t s) {
    const float sl2 = 1.4426950408889634f / sqrtf((float)d);
    const int gxc = (M + 63) / 64, R = B * M, n = gxc * H * B * pl.S;
    float *po = (float *)ws;
    float *pml = po + (size_t)pl.S * R * H * d;
    const bool rag = T % TT != 0;
    const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
#define GR_SPLIT(DD)                                                                            \
    {                                                                                           \
        if (rag) k_cross_split<DD, true><<<n, 256, 0, s>>>(qq, kk, vv, M, H, T, sl2, gxc, n,    \
                                                           pl.S, pl.Ts, R, po, pml);            \
        else k_cross_split<DD, false><<<n, 256, 0, s>>>(qq, kk, vv, M, H, T, sl2, gxc, n, pl.S, \
                                                        pl.Ts, R, po, pml);                     \
        k_cross_merge<DD><<<(R * H + 3) / 4, 256, 0, s>>>(po, pml, (uint16_t *)out, R * H, pl.S); \
    }
    if (d == 32) GR_SPLIT(32)
    else if (d == 64) GR_SPLIT(64)
    else GR_SPLIT(128)
#undef GR_SPLIT
    return hipGetLastError();
}

hipError_t launch_cross_attn(const void *q, const void *k, const void *v, void *out, int B, int M,
                             int H, int T, int d, gr_dtype dt, hipStream_t s) {
    if (dt == GR_F32) {
        const int waves = B * M * H;
        k_cross_f32<<<(waves + 3) / 4, 256, 0, s>>>((const float *)q, (const float *)k,
                                                    (const float *)v, (float *)out, M, H, T, d,
                                                    B * M, 1.0f / sqrtf((float)d));
        return hipGetLastError();
    }
    const float sl2 = 1.4426950408889634f / sqrtf((float)d);
    const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
    uint16_t *oo = (uint16_t *)out;
    // Long key loops amortise each tile's LDS stores and the softmax's
    // per-tile work over 4 row blocks (256 rows) per workgroup when a request
    // has that many rows; short ones take 64 rows per workgroup for more
    // workgroups in flight (d_h = 128 always: more rows would not fit the
    // registers of two waves per SIMD).
    const int rb = T > 2 * TT && d <= 64 ? (M >= 256 ? 4 : 2) : 1;
    const int rows = 64 * rb;
    const int gxc = (M + rows - 1) / rows;
    const int n = gxc * H * B;
    return launch_cross_tiles<false>(qq, kk, vv, oo, M, H, T, d, sl2, gxc, n, rb, T % TT != 0,
                                     JointArgs{}, s);
}

hipError_t launch_joint_attn(const void *q, const void *k, const void *v, const void *k_new,
                             const void *v_new, void *k_pool, void *v_pool, int64_t pool_blocks,
                             int32_t *table, int64_t fresh_base, int B, int M, int H, int T, int d,
                             int t, int L, gr_dtype dt, void *out, hipStream_t s) {
    if (dt == GR_F32) {
        const int waves = B * M * H;
        k_joint_f32<<<(waves + 3) / 4, 256, 0, s>>>(
            (const float *)q, (const float *)k, (const float *)v, (const float *)k_new,
            (const float *)v_new, (float *)k_pool, (float *)v_pool, table, pool_blocks, fresh_base,
            (float *)out, M, H, T, d, B * M, t, L, 1.0f / sqrtf((float)d));
        return hipGetLastError();
    }
    const float sl2 = 1.4426950408889634f / sqrtf((float)d);
    const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
    uint16_t *oo = (uint16_t *)out;
    JointArgs jn;
    jn.k_new = (const uint16_t *)k_new;
    jn.v_new = (const uint16_t *)v_new;
    jn.k_pool = (uint16_t *)k_pool;
    jn.v_pool = (uint16_t *)v_pool;
    jn.table = table;
    jn.pool_blocks = pool_blocks;
    jn.fresh_base = fresh_base;
    jn.t = t;
    jn.L = L;
    // two row blocks per wavefront on long key loops (four cost the beam
    // positions' loop more than they save)
    const bool big = T > 2 * TT && d <= 64;
    const int gxc = (M + (big ? 127 : 63)) / (big ? 128 : 64);
    const int n = gxc * H * B;
    return launch_cross_tiles<true>(qq, kk, vv, oo, M, H, T, d, sl2, gxc, n, big ? 2 : 1,
                                    T % TT != 0, jn, s);
}

hipError_t launch_attn_pair(const void *qx, const void *k_ctx, const void *v_ctx, void *cross_out,
                            int B, int M, int H, int T, int d, const void *q, const void *k_new,
                            const void *v_new, void *k_pool, void *v_pool, int64_t pool_blocks,
                            int32_t *table, int64_t fresh_base, int t, int L, gr_dtype dt,
                            void *self_out, hipStream_t s) {
    const int R = B * M;
    const SelfParams sp = self_params(q, k_new, v_new, k_pool, v_pool, pool_blocks, table,
                                      fresh_base, R, t, L, H, d, dt, self_out);
    const SelfLayout ly = self_layout(sp, dt == GR_BF16);
    if (dt != GR_BF16 || sp.CB != 16 || ly.nch > 4) {   // two launches
        hipError_t e = launch_cross_attn(qx, k_ctx, v_ctx, cross_out, B, M, H, T, d, dt, s);
        if (e != hipSuccess) return e;
        return launch_self_attn(q, k_new, v_new, k_pool, v_pool, pool_blocks, table, fresh_base,
                                R, t, L, H, d, dt, self_out, s);
    }
    const float sl2 = 1.4426950408889634f / sqrtf((float)d);
    const uint16_t *qq = (const uint16_t *)qx, *kk = (const uint16_t *)k_ctx,
                   *vv = (const uint16_t *)v_ctx;
    uint16_t *oo = (uint16_t *)cross_out;
    const bool big = T > 2 * TT && d <= 64;
    const int rows = big ? 128 : 64;
    const int gxc = (M + rows - 1) / rows;
    const int n_cross = gxc * H * B;
    const int srows = 4 * (64 / ly.lpr);
    const dim3 grid(n_cross + (R + srows - 1) / srows);
    const bool rag = T % TT != 0;
#define GR_PAIR_K(DD, RBB, LL, NN)                                                              \
    {                                                                                           \
        if (rag) k_attn_pair<DD, RBB, true, LL, NN><<<grid, 256, 0, s>>>(qq, kk, vv, oo, M, H,  \
                                                                         T, sl2, gxc, n_cross, sp); \
        else k_attn_pair<DD, RBB, false, LL, NN><<<grid, 256, 0, s>>>(qq, kk, vv, oo, M, H, T,  \
                                                                      sl2, gxc, n_cross, sp);   \
    }
#define GR_PAIR(DD, RBB)                                                                        \
    {                                                                                           \
        if (ly.lpr == 16) GR_PAIR_K(DD, RBB, 16, 1)                                             \
        else if (ly.lpr == 32) GR_PAIR_K(DD, RBB, 32, 1)                                        \
        else if (ly.nch <= 1) GR_PAIR_K(DD, RBB, 64, 1)                                         \
        else if (ly.nch <= 2) GR_PAIR_K(DD, RBB, 64, 2)                                         \
        else GR_PAIR_K(DD, RBB, 64, 4)                                                          \
    }
    if (d == 32) {
        if (big) GR_PAIR(32, 2) else GR_PAIR(32, 1)
    } else if (d == 64) {
        if (big) GR_PAIR(64, 2) else GR_PAIR(64, 1)
    } else {
        GR_PAIR(128, 1)
    }
#undef GR_PAIR
#undef GR_PAIR_K
    return hipGetLastError();
}

}  // namespace gr
