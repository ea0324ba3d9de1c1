// Beam-as-query cross-attention on gfx950.
//
// GRACE Section 5.1, eqs 11-14 and Appendix B: the context K, V stay at
// request granularity [B, H, T_ctx, d_h] and the M beam rows of a request are
// that request's query sequence, so one K/V tile load serves every beam of the
// request.  The flattening is request-major (row b*M + m), which is the
// layout bijection of eqs 13-14: no data moves, only the indexing changes.
//
// bf16 path: one workgroup = one (request, head) and up to 128 beam rows
// (4 wavefronts x 2 blocks of 16 rows).  Per 64-key tile, K is staged in LDS
// row-major and V transposed; S^T = K Q^T and O^T += V^T P^T run on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation and an online softmax in
// registers.  Computing the transposed products keeps each lane on one query
// row: its S values are exactly the B operand of the P.V product (the
// key order inside a 32-wide k step is permuted identically for V), and its
// output is a contiguous run of d for one row, stored as 16-byte writes.
// fp32 path (small heads): one wavefront per (row, head), lanes over d.
#include "gr_device.h"
#include "gr_internal.h"

namespace gr {
namespace {

constexpr int TT = 64;          // keys per LDS tile
constexpr int RB = 2;           // 16-row blocks per wavefront
constexpr int ROWS_WG = 4 * RB * 16;
constexpr int PAD = 8;          // bf16 padding per LDS row

union V8 {
    uint4 u;
    bf16x8 b;
};

template <int D>
__global__ __launch_bounds__(256) void k_cross_bf16(const uint16_t *__restrict__ q,
                                                    const uint16_t *__restrict__ K,
                                                    const uint16_t *__restrict__ Vv,
                                                    uint16_t *__restrict__ out, int M, int H,
                                                    int T, float scale_log2) {
    constexpr int NDC = D / 32;   // k steps of S = Q K^T
    constexpr int NDB = D / 16;   // 16-wide blocks of d in O^T
    __shared__ __attribute__((aligned(16))) uint16_t sK[TT][D + PAD];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D][TT + PAD];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, a = lane & 15;
    const int b = blockIdx.z, h = blockIdx.y;
    const int mbase = blockIdx.x * ROWS_WG + wave * RB * 16;
    const size_t kvbase = ((size_t)b * H + h) * (size_t)T * D;

    // Q^T as the B operand: lane (g, a) holds Q[row a][c*32 + g*8 .. +8].
    bf16x8 qf[RB][NDC];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int m = mbase + rb * 16 + a;
#pragma unroll
        for (int c = 0; c < NDC; ++c) {
            V8 t;
            t.u = make_uint4(0, 0, 0, 0);
            if (m < M)
                t.u = *(const uint4 *)(q + (((size_t)b * M + m) * H + h) * D + c * 32 + g * 8);
            qf[rb][c] = t.b;
        }
    }
    f32x4 o[RB][NDB];
    float mrow[RB], lpart[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        mrow[rb] = -INFINITY;
        lpart[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int t0 = 0; t0 < T; t0 += TT) {
        __syncthreads();
        for (int idx = tid; idx < TT * (D / 8); idx += 256) {
            const int key = idx / (D / 8), dc = idx % (D / 8);
            uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
            if (t0 + key < T) {
                kv = *(const uint4 *)(K + kvbase + (size_t)(t0 + key) * D + dc * 8);
                vv = *(const uint4 *)(Vv + kvbase + (size_t)(t0 + key) * D + dc * 8);
            }
            *(uint4 *)&sK[key][dc * 8] = kv;
            const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sVt[dc * 8 + 2 * e][key] = (uint16_t)(w[e] & 0xFFFFu);
                sVt[dc * 8 + 2 * e + 1][key] = (uint16_t)(w[e] >> 16);
            }
        }
        __syncthreads();

#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            // S^T block kb: lane holds S[row a][key t0 + kb*16 + g*4 + i].
            f32x4 s[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NDC; ++c) {
                    V8 ka;
                    ka.u = *(const uint4 *)&sK[kb * 16 + a][c * 32 + g * 8];
                    s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka.b, qf[rb][c], s[kb], 0, 0, 0);
                }
            }
            float tmax = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s[kb][i] * scale_log2;
                    if (t0 + kb * 16 + g * 4 + i >= T) v = -INFINITY;
                    s[kb][i] = v;
                    tmax = fmaxf(tmax, v);
                }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float mnew = fmaxf(mrow[rb], tmax);
            const float alpha = __builtin_amdgcn_exp2f(mrow[rb] - mnew);
            mrow[rb] = mnew;
            float lsum = 0.0f;
            uint32_t pk[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float pv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint16_t hb = f32_to_bf16(__builtin_amdgcn_exp2f(s[kb][i] - mnew));
                    pv[i] = bf16_to_f32(hb);   // the weight the product uses
                    lsum += pv[i];
                }
                pk[kb][0] = pack_bf16x2(pv[0], pv[1]);
                pk[kb][1] = pack_bf16x2(pv[2], pv[3]);
            }
            lpart[rb] = lpart[rb] * alpha + lsum;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[rb][db] *= alpha;
            // O^T += V^T P^T, k step over keys of sub-blocks (2pc, 2pc+1):
            // slot g*8+i <-> key (2pc)*16 + g*4 + i (i < 4),
            //                    (2pc+1)*16 + g*4 + i-4 (i >= 4).
#pragma unroll
            for (int pc = 0; pc < 2; ++pc) {
                V8 pb;
                pb.u = make_uint4(pk[2 * pc][0], pk[2 * pc][1], pk[2 * pc + 1][0], pk[2 * pc + 1][1]);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    // A row a <-> d = (a/4)*4*NDB + db*4 + a%4
                    const int d = (a >> 2) * (4 * NDB) + db * 4 + (a & 3);
                    const uint2 lo = *(const uint2 *)&sVt[d][(2 * pc) * 16 + g * 4];
                    const uint2 hi = *(const uint2 *)&sVt[d][(2 * pc + 1) * 16 + g * 4];
                    V8 va;
                    va.u = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.b, pb.b, o[rb][db], 0, 0, 0);
                }
            }
        }
    }

    // Lane (g, a) holds O[row a][d = g*4*NDB + db*4 + i].
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        float lt = lpart[rb];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        const float inv = 1.0f / lt;
        const int m = mbase + rb * 16 + a;
        if (m >= M) continue;
        uint32_t w[2 * NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            w[2 * db] = pack_bf16x2(o[rb][db][0] * inv, o[rb][db][1] * inv);
            w[2 * db + 1] = pack_bf16x2(o[rb][db][2] * inv, o[rb][db][3] * inv);
        }
        uint16_t *dst = out + (((size_t)b * M + m) * H + h) * D + g * 4 * NDB;
#pragma unroll
        for (int c = 0; c < NDB / 2; ++c)
            *(uint4 *)(dst + c * 8) = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
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

}  // namespace

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
    dim3 grid((M + ROWS_WG - 1) / ROWS_WG, H, B);
    const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
    uint16_t *oo = (uint16_t *)out;
    if (d == 32) k_cross_bf16<32><<<grid, 256, 0, s>>>(qq, kk, vv, oo, M, H, T, sl2);
    else if (d == 64) k_cross_bf16<64><<<grid, 256, 0, s>>>(qq, kk, vv, oo, M, H, T, sl2);
    else k_cross_bf16<128><<<grid, 256, 0, s>>>(qq, kk, vv, oo, M, H, T, sl2);
    return hipGetLastError();
}

}  // namespace gr
