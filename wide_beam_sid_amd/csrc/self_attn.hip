// Paged short-prefix self-attention on gfx950.
//
// GRACE Section 5.2 (each beam row attends only to its own cached prefix:
// the block-diagonal mask, not a causal one), Section 5.2 "kernel fusion"
// (the kernel consumes q/k/v, writes the current token's k, v into the cache,
// gathers the prefix and returns the output) and Section 5.3 / Section 3.3
// (flat KV pool of one-token blocks addressed through the block table P;
// reorder copies block ids only).  GR-Inference's CUDA-core beam attention
// (K2) makes the same choice of plain FMA over matrix units for such short,
// gathered sequences.
//
// One wavefront per beam row.  A row's H*d_h elements are spread over the 64
// lanes in 8-byte chunks (4 bf16 or 2 fp32 per lane per chunk), so every load
// and store of q, k, v, out and of a gathered pool block is one fully
// coalesced wavefront access; the d_h/VEC lanes of a head reduce their dot
// products with xor shuffles.  The prefix block ids are read in one load,
// the blocks' K/V are gathered in batches with all loads of a batch in
// flight, and positions are consumed with an online softmax.
#include "self_attn_body.h"

namespace gr {
namespace {

template <bool BF16, int NCH>
__global__ __launch_bounds__(256) void k_self_attn(SelfParams p) {
    self_attn_rows<BF16, NCH>(p, blockIdx.x);
}

template <bool BF16>
hipError_t dispatch(const SelfParams &p, hipStream_t s) {
    constexpr int VEC = Chunk<BF16>::VEC;
    const int nch = (p.E / VEC + 63) / 64;
    dim3 grid((p.R + 3) / 4);
    if (nch <= 1) k_self_attn<BF16, 1><<<grid, 256, 0, s>>>(p);
    else if (nch <= 2) k_self_attn<BF16, 2><<<grid, 256, 0, s>>>(p);
    else if (nch <= 4) k_self_attn<BF16, 4><<<grid, 256, 0, s>>>(p);
    else if (nch <= 8) k_self_attn<BF16, 8><<<grid, 256, 0, s>>>(p);
    else k_self_attn<BF16, 16><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_self_attn(const void *q, const void *k_new, const void *v_new, void *k_pool,
                            void *v_pool, int64_t pool_blocks, int32_t *table,
                            int64_t fresh_base, int R, int t, int L, int H, int d, gr_dtype dt,
                            void *out, hipStream_t s) {
    const SelfParams p = self_params(q, k_new, v_new, k_pool, v_pool, pool_blocks, table,
                                     fresh_base, R, t, L, H, d, dt, out);
    if (dt == GR_BF16) return dispatch<true>(p, s);
    return dispatch<false>(p, s);
}

}  // namespace gr
