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
// A beam row's H*d_h elements are spread over 16, 32 or 64 lanes in 16-byte
// pieces (8 bf16 or 4 fp32 per lane; 8-byte pieces when a head is narrower
// than 16 bytes), so a wavefront holds one to four rows and every load and
// store of q, k, v, out and of a gathered pool block is a coalesced access.
// The lanes of a head sum their dot products with DPP butterflies (8-lane
// heads) or permutes.  A row's prefix block ids are read per batch of
// positions, the blocks' K/V gathered with all loads of a batch in flight,
// and the positions consumed with an online softmax.
#include "self_attn_body.h"

namespace gr {
namespace {

template <bool BF16, int CB, int LPR, int NCH, int GC>
__global__ __launch_bounds__(256) void k_self_attn(SelfParams p) {
    self_attn_rows<BF16, CB, LPR, NCH, GC>(p, blockIdx.x);
}

// GC: 8 lanes per head (bf16 heads of 64 in 16-byte pieces) summed with
// compile-time DPP steps; 0 for any other width, summed by permutes
template <bool BF16, int CB, int LPR, int NCH>
hipError_t go(const SelfParams &p, hipStream_t s) {
    constexpr int rows = self_rows_wg<LPR>();
    const dim3 grid((p.R + rows - 1) / rows);
    if (p.G == 8) k_self_attn<BF16, CB, LPR, NCH, 8><<<grid, 256, 0, s>>>(p);
    else k_self_attn<BF16, CB, LPR, NCH, 0><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
}

template <bool BF16>
hipError_t dispatch(const SelfParams &p, hipStream_t s) {
    const SelfLayout ly = self_layout(p, BF16);
    if (p.CB == 8) {
        if (ly.nch <= 1) return go<BF16, 8, 64, 1>(p, s);
        if (ly.nch <= 2) return go<BF16, 8, 64, 2>(p, s);
        if (ly.nch <= 4) return go<BF16, 8, 64, 4>(p, s);
        if (ly.nch <= 8) return go<BF16, 8, 64, 8>(p, s);
        return go<BF16, 8, 64, 16>(p, s);
    }
    if (ly.lpr == 16) return go<BF16, 16, 16, 1>(p, s);
    if (ly.lpr == 32) return go<BF16, 16, 32, 1>(p, s);
    if (ly.nch <= 1) return go<BF16, 16, 64, 1>(p, s);
    if (ly.nch <= 2) return go<BF16, 16, 64, 2>(p, s);
    if (ly.nch <= 4) return go<BF16, 16, 64, 4>(p, s);
    return go<BF16, 16, 64, 8>(p, s);
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
