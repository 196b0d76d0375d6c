// gemm_bf16.hip — the dense products of the attention layer with its projections, on gfx950 bf16
// MFMA: q/k/v = x W (hidden -> heads) and out = v_scale * attn W_o (heads -> hidden).
//
// Pages: "Add Xiaomi MiMo-V2", section "Additional useful info" (the QK and V head dims are
// decoupled, so the projections have different widths; values are rescaled by
// sqrt(hidden / (heads * v_head_dim)), which by linearity rides on the output product's scale);
// "add Xiaomi MiMo v2 (mimo_v2_flash)", sections "Architecture, verified against upstream" and
// "Implementation plan" (partial rotation of the leading dims of each key, rotating cache of the
// sliding layers).
//
// C[M, N] = alpha * A[M, K] * B[K, N], A and B row-major bf16, fp32 accumulation, C rounded once to
// bf16.  Shape of the computation:
//   * a workgroup of 8 waves (two per SIMD) computes a 256 x 256 tile of C; wave w owns rows
//     64 (w % 4) .. + 63 (two 32-row blocks) and columns 128 (w / 4) .. + 127 (four 32-column
//     blocks): 8 accumulators of 32 x 32;
//   * it computes C^T: v_mfma_f32_32x32x16_bf16 with B^T as the A operand (32 columns of C x 16 k,
//     read transposed from the LDS B tile by ds_read_b64_tr_b16) and A^T as the B operand (32 rows
//     of C, 8 consecutive k per lane, read straight from the LDS A tile), so that each lane ends
//     with one row of C and, per block, four groups of four consecutive columns (8-byte stores);
//   * A (256 x 32) and B (32 x 256) tiles stream through a 4-stage LDS ring (128 KiB) filled by
//     global_load_lds_dwordx4, three tiles ahead of the one being computed (with 64-deep tiles
//     and two stages, one tile ahead, each tile's copy latency sat on the products' path); A rows
//     (64 bytes) are swizzled at 16-byte granularity (chunk c of row r at c ^ ((r >> 2) & 3)),
//     B rows as chunk c at c ^ 4 (r & 3), so that both operand reads are conflict-free;
//   * epilogues: plain (C = alpha * acc); key projection (the rotation of the leading 64 dims of
//     each key head applied to the fp32 accumulators, the rotated key stored in the attention's
//     [B, Hkv, S, dqk] layout and into the KV cache: linear slot = position, ring slot =
//     position % window for the last `window` tokens, bf16 or e4m3 codes of the fp32 value);
//     value projection (plain store plus the cache store).
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mimo {
namespace {

constexpr int GBM = 256, GBN = 256, GBK = 32, GSTAGES = 4, GW = 8;
constexpr int A_TILE = GBM * GBK * 2;   // bytes
constexpr int B_TILE = GBK * GBN * 2;
constexpr int A_DMA = A_TILE / 1024 / GW;   // 1-KiB DMA instructions per wave per tile
constexpr int B_DMA = B_TILE / 1024 / GW;

__global__ __launch_bounds__(GW * 64) void gemm_bf16_kernel(const GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[GSTAGES * (A_TILE + B_TILE)];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    // the product this workgroup belongs to (the grid holds the tiles of every part in turn)
    int bid = (int)blockIdx.x, pi = 0;
    if (a.nparts > 1 && bid >= a.part[0].tiles) {
        bid -= a.part[0].tiles;
        pi = 1;
        if (a.nparts > 2 && bid >= a.part[1].tiles) {
            bid -= a.part[1].tiles;
            pi = 2;
        }
    }
    const uint16_t* const Bm = a.part[pi].B;
    uint16_t* const Cm = a.part[pi].C;
    void* const cache = a.part[pi].cache;
    const int64_t ldb = a.part[pi].ldb, ldc = a.part[pi].ldc;
    const int N = a.part[pi].N, epi = a.part[pi].epilogue;
    const float code_inv = a.part[pi].code_inv;
    const int ntn = (N + GBN - 1) / GBN;
    // consecutive workgroups walk the column tiles of one row tile (the A tile stays in L2)
    const int tm = bid / ntn, tn = bid % ntn;
    const int m0 = tm * GBM, n0 = tn * GBN;
    const int wm = wave & 3, wn = wave >> 2;   // wave's 64-row and 128-column slice
    const int nk = a.K / GBK;

    // ---- DMA sources: LDS 16-byte slot P of this wave's instruction i holds A row P / 4, logical
    //      chunk (P % 4) ^ ((row >> 2) & 3); B row P / 32, chunk (P % 32) ^ 4 (row & 3).
    constexpr int ACH = GBK / 8;   // 16-byte chunks per A row
    const uint16_t* ap[A_DMA];
    const uint16_t* bp[B_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int P = (wave * A_DMA + i) * 64 + lane;
        const int row = P / ACH, phys = P % ACH;
        const int m = min(m0 + row, a.M - 1);
        ap[i] = a.A + (int64_t)m * a.lda + ((phys ^ ((row >> 2) & 3)) * 8);
    }
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const int P = (wave * B_DMA + i) * 64 + lane;
        const int row = P / 32, phys = P % 32;
        const int n = min(n0 + ((phys ^ ((row & 3) << 2)) * 8), N - 8);
        bp[i] = Bm + (int64_t)row * ldb + n;
    }
    const uint32_t lds0 = (uint32_t)(size_t)(lds_u8_t*)smem;
    auto issue = [&](int t, int st) {
        const uint32_t ast = lds0 + st * A_TILE;
        const uint32_t bst = lds0 + GSTAGES * A_TILE + st * B_TILE;
        const int64_t dk = (int64_t)t * GBK;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) dma16(ap[i] + dk, ast + (wave * A_DMA + i) * 1024);
#pragma unroll
        for (int i = 0; i < B_DMA; ++i) dma16(bp[i] + dk * ldb, bst + (wave * B_DMA + i) * 1024);
    };
#pragma unroll
    for (int t = 0; t < GSTAGES - 1; ++t)
        if (t < nk) issue(t, t);

    // ---- per-lane LDS read offsets (bytes within a stage)
    // A^T operand, row block mb: row r = 64 wave + 32 mb + l32, logical chunk 2 kk + g
    int a_rd[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) a_rd[mb] = (64 * wm + 32 * mb + l32) * (GBK * 2);
    const int aswz = (l32 >> 2) & 3;   // ((row >> 2) & 3) of every row this lane reads
    // B^T operand, column block nb: ds_read_b64_tr_b16 hands lane j of a 16-lane group
    // B[k0 + t][n0 + j] (t < 4) when it points at B[k0 + j/4][n0 + 4 (j % 4)]; lane group g takes
    // k rows 8g .. 8g + 3 and, in a second read, 8g + 4 .. 8g + 7 (the 8 consecutive k that the
    // A^T operand holds for that group)
    const int qsel = lane >> 4, jsel = lane & 15;
    const int brow = 8 * (qsel >> 1) + (jsel >> 2);
    int b_rd[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        b_rd[nb] = GSTAGES * A_TILE + brow * (GBN * 2) +
                   16 * (4 * ((4 * wn + nb) ^ ((jsel >> 2) & 3)) + 2 * (qsel & 1) + ((jsel & 3) >> 1)) +
                   8 * (jsel & 1);
        asm volatile("" : "+v"(b_rd[nb]));
    }

    f32x16 acc[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x16{};

    for (int t = 0; t < nk; ++t) {
        const int st = t % GSTAGES;
        // tile t has landed once at most the later tiles' copies are outstanding (this wave's
        // copies complete in order)
        if (t + 2 < nk) wait_vmcnt<2 * (A_DMA + B_DMA)>();
        else if (t + 1 < nk) wait_vmcnt<A_DMA + B_DMA>();
        else wait_vmcnt<0>();
        block_sync_lds();   // tile t is in LDS for every wave; stage (t - 1) % 4 is free
        if (t + GSTAGES - 1 < nk) issue(t + GSTAGES - 1, (t + GSTAGES - 1) % GSTAGES);
        const uint8_t* as = smem + st * A_TILE;
        const uint8_t* bs = smem + st * B_TILE;   // + b_rd, which holds the B area's base
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) {
            bf16x8 At[2], Bt[4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                At[mb] = *(const bf16x8*)(as + a_rd[mb] + 16 * ((2 * kk + g) ^ aswz));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const uint8_t* p = bs + b_rd[nb] + 16 * kk * (GBN * 2);
                const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
                const bf16x4 v1 =
                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * GBN * 2));
                Bt[nb] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = mfma32x32x16(Bt[nb], At[mb], acc[mb][nb]);
        }
    }

    // ---- epilogue.  acc[mb][nb][i] = C[m][n], m = m0 + 64 wave + 32 mb + l32,
    //      n = n0 + 32 nb + 8 (i / 4) + 4 g + (i % 4)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int m = m0 + 64 * wm + 32 * mb + l32;
        if (m >= a.M) continue;
        float v[4][16];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int i = 0; i < 16; ++i) v[nb][i] = acc[mb][nb][i] * a.alpha;
        int32_t pos = 0, bseq = 0, tok = 0;
        if (epi != kGemmPlain) {
            bseq = m / a.S;
            tok = m - bseq * a.S;
            pos = a.start_pos[bseq] + tok;
        }
        if (epi == kGemmKey) {
            // the head whose first dims lie in this tile: heads start at multiples of dqk (192),
            // so at most one start falls in a 128-column tile, at offset 0 or 64; its dims
            // [0, 64) are blocks (hb, hb + 1) and pair d (block hb) with d + 32 (block hb + 1)
            const int nw0 = n0 + 128 * wn;
            const int hs = ((nw0 + a.dqk - 1) / a.dqk) * a.dqk;   // first head start >= nw0
            if (a.rope_dims > 0 && hs < nw0 + 128 && hs < N) {
                const int hb = (hs - nw0) / 32;   // 0 or 2 (uniform)
#pragma unroll
                for (int pb = 0; pb < 3; pb += 2) {
                    if (hb != pb) continue;
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int d = 8 * (i >> 2) + 4 * g + (i & 3);
                        float c, s;
                        rope_cos_sin_rev(pos, a.omega_rev[d], c, s);
                        const float x = v[pb][i], y = v[pb + 1][i];
                        v[pb][i] = x * c - y * s;
                        v[pb + 1][i] = y * c + x * s;
                    }
                }
            }
        }
        const bool store_cache = epi != kGemmPlain && cache && tok >= a.cache_i0;
        const int slot = a.ring_window > 0 ? pos % a.ring_window : pos;
        const bool slot_ok = store_cache && slot >= 0 && slot < a.cap;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int n = n0 + 128 * wn + 32 * nb + 8 * q4 + 4 * g;
                if (n >= N) continue;
                const float* x = &v[nb][4 * q4];
                const u32x2 w = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
                if (epi == kGemmPlain) {
                    *(u32x2*)(Cm + (int64_t)m * ldc + n) = w;
                } else {
                    // key: the rotated key in the attention's [B, Hkv, S, dqk] layout;
                    // value: row-major [B * S, Hkv * dv]
                    const int hd = epi == kGemmKey ? a.dqk : a.dv;
                    const int kvh = n / hd, d = n - kvh * hd;
                    if (epi == kGemmKey)
                        *(u32x2*)(Cm + (((int64_t)bseq * a.heads + kvh) * a.S + tok) * hd + d) = w;
                    else
                        *(u32x2*)(Cm + (int64_t)m * ldc + n) = w;
                    if (slot_ok) {
                        const int64_t crow = ((int64_t)bseq * a.heads + kvh) * a.cap + slot;
                        if (a.cache_fp8) {
                            // codes of the fp32 rotated key; of the value's bf16 rounding (the
                            // value the attention reads)
                            float y[4];
#pragma unroll
                            for (int t = 0; t < 4; ++t) {
                                const float xv = epi == kGemmKey
                                                     ? x[t]
                                                     : __uint_as_float((t & 1) ? (w[t >> 1] & 0xffff0000u)
                                                                               : (w[t >> 1] << 16));
                                y[t] = fminf(fmaxf(xv * code_inv, -448.0f), 448.0f);
                            }
                            int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                            c = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c, true);
                            *(uint32_t*)((uint8_t*)cache + crow * hd + d) = (uint32_t)c;
                        } else {
                            *(u32x2*)((uint16_t*)cache + crow * hd + d) = w;
                        }
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
    if (a.M == 0 || a.nparts < 1 || a.nparts > 3) return a.M == 0 ? hipSuccess : hipErrorInvalidValue;
    if (a.K % GBK || a.K < GBK) return hipErrorInvalidValue;
    GemmArgs k = a;
    int64_t tiles = 0;
    for (int p = 0; p < a.nparts; ++p) {
        if (a.part[p].N < 8 || a.part[p].N % 8) return hipErrorInvalidValue;
        const int64_t t = (int64_t)((a.M + GBM - 1) / GBM) * ((a.part[p].N + GBN - 1) / GBN);
        if (t > 0x7fffffff) return hipErrorInvalidConfiguration;
        k.part[p].tiles = (int32_t)t;
        tiles += t;
    }
    if (tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    gemm_bf16_kernel<<<dim3((unsigned)tiles), GW * 64, 0, st>>>(k);
    return hipGetLastError();
}

}  // namespace mimo
