// Tiled bf16 GEMM for gfx950 with fused output-tile epilogues.
//
// One GPU's share of the ParallelKittens kernels is a single-GPU tiled GEMM plus a small
// epilogue ("Loads and Loads of Fluffy Kittens" summary, Key claims: tiling is kept and each
// multi-GPU kernel adds little device code on top of the single-GPU kernel; Method: the output
// tile of the GEMM is exactly what is sent and atomically added at the destination).  The
// single-GPU core follows the tile / block / grid structure the ThunderKittens article describes
// (tiles staged through swizzled on-chip memory, multi-stage buffering, L2-aware block order),
// re-derived for CDNA4:
//
//  * MFMA v_mfma_f32_32x32x16_bf16: every wave owns a (FM*32) x (FN*32) accumulator block held in
//    registers; operands come from LDS as 16-byte reads (8 consecutive k per lane).
//  * Operand staging: A (M x K, k-contiguous) is copied HBM -> registers -> LDS unchanged.  B
//    (K x N row-major, n-contiguous) is loaded as 8x8 sub-blocks and transposed in registers so
//    that LDS holds B^T (n rows, k-contiguous), the layout the MFMA B operand wants.
//  * LDS rows of BK bf16 are split in 16-byte chunks whose position is XOR-swizzled with the row
//    index (the article's bank = column XOR (row >> shift) scheme, widened so that 8 or 16
//    consecutive rows of a 16-byte read land on distinct banks).
//  * Two LDS stages: global loads of k-step t+1 are in flight while the MFMAs of step t run; one
//    workgroup barrier per k-step.
//  * Grid: workgroups are dealt round-robin to the 8 XCDs; block ids are remapped so that each XCD
//    works on one contiguous run of logical tiles, and logical tiles are rastered in groups of
//    tile rows, so operand panels are reused from that XCD's L2.
#include "pk_internal.h"

namespace pk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MIN_WG_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int CPR = BK / 8;  // 16-byte chunks per LDS row
    static constexpr int A_LOADS = BM * CPR / NT;
    static constexpr int B_SUBS = (BK / 8) * (BN / 8);  // 8 (k) x 8 (n) sub-blocks
    static constexpr int B_LOADS = (B_SUBS + NT - 1) / NT;
    static constexpr int ROW_BYTES = BK * 2;
    static constexpr int LDS_A = BM * ROW_BYTES;
    static constexpr int LDS_B = BN * ROW_BYTES;
    static constexpr int LDS_STAGE = LDS_A + LDS_B;
    static constexpr int LDS_BYTES = 2 * LDS_STAGE;
    static constexpr int MIN_WG = MIN_WG_;
    static_assert((BM * CPR) % NT == 0, "A chunks must split evenly over threads");
    static_assert(NT % CPR == 0, "each thread keeps one k-chunk of A");
    static_assert(BK == 32 || BK == 64, "LDS swizzle defined for 64- and 128-byte rows");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles are made of 32x32 MFMA blocks");
};

using Cfg256x256 = Cfg<256, 256, 64, 2, 2, 1>;
using Cfg256x128 = Cfg<256, 128, 64, 2, 2, 1>;
using Cfg256x128x2 = Cfg<256, 128, 32, 2, 2, 2>;
using Cfg128x128 = Cfg<128, 128, 64, 2, 2, 1>;

TileShape tile_shape(TileCfgId cfg) {
    switch (cfg) {
        case CFG_256x256: return {256, 256};
        case CFG_256x128: return {256, 128};
        case CFG_256x128_2WG: return {256, 128};
        default: return {128, 128};
    }
}

// ------------------------------------------------------------------------------------------------
// Small device helpers
// ------------------------------------------------------------------------------------------------

// 16-byte chunk position inside an LDS row, XOR-swizzled with the row.
template <int CPR>
__device__ __forceinline__ int lds_offset(int row, int chunk) {
    int s;
    if constexpr (CPR == 8)
        s = (row ^ (row >> 3)) & 7;
    else
        s = ((row >> 1) ^ (row >> 3)) & 3;
    return row * (CPR * 16) + ((chunk ^ s) << 4);
}

// Round to nearest even, fp32 -> bf16 bits (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Pick table[i] with a chain of selects (keeps kernel-argument tables out of scratch memory).
template <typename T>
__device__ __forceinline__ T pick(const T (&table)[PK_MAX_PARTS], int i) {
    T r = table[0];
#pragma unroll
    for (int j = 1; j < PK_MAX_PARTS; ++j) r = (i == j) ? table[j] : r;
    return r;
}

// Hardware block id -> logical tile id.  Blocks are dealt to the 8 XCDs round-robin
// (block b runs on XCD b % 8); XCD x receives logical tiles [x*q + min(x, r), ...) in launch
// order, so neighbouring logical tiles share an L2.  Returns false for surplus blocks.
__device__ __forceinline__ bool xcd_remap(int b, int total, int& L) {
    const int x = b & 7, s = b >> 3;
    const int q = total >> 3, r = total & 7;
    const int cnt = q + (x < r ? 1 : 0);
    if (s >= cnt) return false;
    L = x * q + (x < r ? x : r) + s;
    return true;
}

// ------------------------------------------------------------------------------------------------
// The kernel
// ------------------------------------------------------------------------------------------------

template <class C, bool GROUPED, int EPI>
__global__ __launch_bounds__(C::NT, C::MIN_WG) void gemm_tile_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) char lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wy = wave / C::WAVES_N;
    const int wx = wave % C::WAVES_N;

    const int64_t M = p.M, N = p.N, K = p.K;
    const int tiles_n = (int)((N + C::BN - 1) / C::BN);

    // ---- which output tile ----------------------------------------------------------------
    int64_t row0, row_end, col0;
    const uint16_t* Bm = p.B;
    int L;
    if constexpr (GROUPED) {
        const int num_local = p.num_local;
        const int mt_total = p.tile_offsets[num_local];
        if (!xcd_remap(blockIdx.x, mt_total * tiles_n, L)) return;
        // expert e: largest e with tile_offsets[e] * tiles_n <= L (empty experts are skipped)
        int lo = 0, hi = num_local;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.tile_offsets[mid] * tiles_n <= L) lo = mid; else hi = mid;
        }
        const int e = lo;
        const int t0 = p.tile_offsets[e];
        const int me = p.tile_offsets[e + 1] - t0;
        const int local = L - t0 * tiles_n;
        const int tn = local / me, mt = local - tn * me;  // expert-major, then n, then m
        row0 = (int64_t)p.offsets[e] + (int64_t)mt * C::BM;
        row_end = p.offsets[e + 1];
        col0 = (int64_t)tn * C::BN;
        Bm = p.B + (int64_t)e * p.b_stride;
    } else {
        const int tiles_m = (int)((M + C::BM - 1) / C::BM);
        if (!xcd_remap(blockIdx.x, tiles_m * tiles_n, L)) return;
        const int gm_rows = p.group_m;
        const int per_group = gm_rows * tiles_n;
        const int g = L / per_group, li = L - g * per_group;
        const int first = g * gm_rows;
        const int gm = min(tiles_m - first, gm_rows);
        int tm = first + li % gm;
        const int tn = li / gm;
        tm += p.rot_tile_rows;
        if (tm >= tiles_m) tm -= tiles_m;
        row0 = (int64_t)tm * C::BM;
        row_end = M;
        col0 = (int64_t)tn * C::BN;
    }

    // ---- per-thread operand sources (fixed for the whole k-loop) ----------------------------
    const int a_kc = tid % C::CPR;  // this thread's 16-byte k-chunk of A
    const uint16_t* a_src[C::A_LOADS];
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
        const int rl = (i * C::NT + tid) / C::CPR;
        int64_t r = row0 + rl;
        if (r >= row_end) r = row0;  // masked row: read a valid one, never stored
        const uint16_t* src;
        if constexpr (GROUPED) {
            const int64_t token = p.perm[r] / p.top_k;
            src = p.a_ptr[0] + token * p.lda;
        } else {
            if (p.num_chunks == 1) {
                src = p.a_ptr[0] + r * p.lda;
            } else {
                const int c = (int)(r / p.chunk_rows);
                src = pick(p.a_ptr, c) + (r - (int64_t)c * p.chunk_rows) * p.lda;
            }
        }
        a_src[i] = src + a_kc * 8;
    }
    const uint16_t* b_src[C::B_LOADS];
    int b_kg[C::B_LOADS], b_ng[C::B_LOADS];
    bool b_on[C::B_LOADS];
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j) {
        const int s = j * C::NT + tid;
        b_on[j] = s < C::B_SUBS;
        const int ss = b_on[j] ? s : 0;
        b_kg[j] = ss / (C::BN / 8);
        b_ng[j] = ss % (C::BN / 8);
        int64_t col = col0 + b_ng[j] * 8;
        if (col >= N) col = 0;  // masked columns: read valid memory, never stored
        b_src[j] = Bm + (int64_t)(b_kg[j] * 8) * p.ldb + col;
    }

    u32x4 ra[C::A_LOADS];
    u32x4 rb[C::B_LOADS][8];

    auto load_step = [&](int64_t k0, bool tail) {
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            if (!tail || k0 + a_kc * 8 < K)
                ra[i] = *(const u32x4*)(a_src[i] + k0);
            else
                ra[i] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < C::B_LOADS; ++j) {
            if (!b_on[j]) continue;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int64_t k = k0 + b_kg[j] * 8 + r;
                if (!tail || k < K)
                    rb[j][r] = *(const u32x4*)(b_src[j] + (k0 + r) * p.ldb);
                else
                    rb[j][r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    auto store_step = [&](int stage) {
        char* sA = lds + stage * C::LDS_STAGE;
        char* sB = sA + C::LDS_A;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            const int rl = (i * C::NT + tid) / C::CPR;
            *(u32x4*)(sA + lds_offset<C::CPR>(rl, a_kc)) = ra[i];
        }
#pragma unroll
        for (int j = 0; j < C::B_LOADS; ++j) {
            if (!b_on[j]) continue;
            // rb[j][k] holds B[k][n0..n0+7] as 4 words of two bf16 (n even low, n odd high);
            // emit, for each n, the 8 consecutive k as one 16-byte chunk.
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const int d = n >> 1;
                u32x4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = rb[j][2 * e][d], hi = rb[j][2 * e + 1][d];
                    o[e] = (n & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                   : ((lo & 0xffffu) | (hi << 16));
                }
                *(u32x4*)(sB + lds_offset<C::CPR>(b_ng[j] * 8 + n, b_kg[j])) = o;
            }
        }
    };

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

    auto compute_step = [&](int stage) {
        const char* sA = lds + stage * C::LDS_STAGE;
        const char* sB = sA + C::LDS_A;
#pragma unroll
        for (int kk = 0; kk < C::BK / 16; ++kk) {
            const int ch = kk * 2 + (lane >> 5);
            bf16x8 af[C::FM], bfr[C::FN];
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
                af[fm] = *(const bf16x8*)(sA + lds_offset<C::CPR>(wy * C::WTM + fm * 32 + (lane & 31), ch));
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
                bfr[fn] = *(const bf16x8*)(sB + lds_offset<C::CPR>(wx * C::WTN + fn * 32 + (lane & 31), ch));
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
        }
    };

    // ---- k-loop: loads of step t+1 in flight during the MFMAs of step t ---------------------
    const int64_t nk = (K + C::BK - 1) / C::BK;
    if (nk > 0) {
        load_step(0, C::BK > K);
        store_step(0);
        __syncthreads();
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int stage = (int)(kt & 1);
            const bool more = kt + 1 < nk;
            if (more) load_step((kt + 1) * C::BK, (kt + 2) * C::BK > K);
            compute_step(stage);
            if (more) store_step(stage ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogue ----------------------------------------------------------------------------
    // Accumulator element r of block (fm, fn) in lane l sits at tile row
    // fm*32 + (r/4)*8 + (l/32)*4 + r%4 and tile column fn*32 + l%32 of this wave's sub-tile.
    const int lrow = (lane >> 5) * 4;
    const int lcol = lane & 31;
    const int64_t wrow0 = row0 + wy * C::WTM;
    const int64_t wcol0 = col0 + wx * C::WTN;

    if constexpr (EPI == EPI_STORE_BF16 || EPI == EPI_STORE_F32) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) {
                const int64_t col = wcol0 + fn * 32 + lcol;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t row = wrow0 + fm * 32 + (r >> 2) * 8 + lrow + (r & 3);
                    if (row < row_end && col < N) {
                        if constexpr (EPI == EPI_STORE_BF16)
                            ((uint16_t*)p.C)[row * p.ldc + col] = (uint16_t)bf16_rne(acc[fm][fn][r]);
                        else
                            ((float*)p.C)[row * p.ldc + col] = acc[fm][fn][r];
                    }
                }
            }
    } else {
        // Reduction into the destination.  With several shards, shard_rows is a multiple of 32
        // and tile rows start at multiples of 32, so every 32-row accumulator block lies in one
        // shard and its destination base is uniform across the wave.
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int64_t brow = wrow0 + fm * 32;  // first row of this 32-row block
            if (brow < M) {
                const int s = p.num_shards == 1 ? 0 : (int)(brow / p.shard_rows);
                float* const dbase = pick(p.d_ptr, s) + (brow - (int64_t)s * p.shard_rows) * p.ldd;
                if constexpr (EPI == EPI_OWNER_F32) {
                    // read the whole destination block first, then add and write it back
                    float cur[C::FN][16];
#pragma unroll
                    for (int fn = 0; fn < C::FN; ++fn) {
                        const int64_t col = wcol0 + fn * 32 + lcol;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int rr = (r >> 2) * 8 + lrow + (r & 3);
                            const bool in = (brow + rr < M) && (col < N);
                            cur[fn][r] = in ? dbase[(int64_t)rr * p.ldd + col] : 0.0f;
                        }
                    }
#pragma unroll
                    for (int fn = 0; fn < C::FN; ++fn) {
                        const int64_t col = wcol0 + fn * 32 + lcol;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int rr = (r >> 2) * 8 + lrow + (r & 3);
                            if ((brow + rr < M) && (col < N))
                                dbase[(int64_t)rr * p.ldd + col] = cur[fn][r] + acc[fm][fn][r];
                        }
                    }
                } else {
#pragma unroll
                    for (int fn = 0; fn < C::FN; ++fn) {
                        const int64_t col = wcol0 + fn * 32 + lcol;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int rr = (r >> 2) * 8 + lrow + (r & 3);
                            if ((brow + rr < M) && (col < N))
                                __hip_atomic_fetch_add(dbase + (int64_t)rr * p.ldd + col,
                                                       acc[fm][fn][r], __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------------------------------------
// Host-side launchers
// ------------------------------------------------------------------------------------------------

template <class C, bool GROUPED, int EPI>
static hipError_t launch_one(const GemmArgs& a, int64_t tiles, hipStream_t stream) {
    if (tiles <= 0) return hipSuccess;
    const int64_t grid = (tiles + 7) / 8 * 8;
    hipLaunchKernelGGL((gemm_tile_kernel<C, GROUPED, EPI>), dim3((unsigned)grid), dim3(C::NT), 0,
                       stream, a);
    return hipGetLastError();
}

template <class C, bool GROUPED>
static hipError_t launch_epi(const GemmArgs& a, Epi epi, int64_t tiles, hipStream_t stream) {
    switch (epi) {
        case EPI_STORE_BF16: return launch_one<C, GROUPED, EPI_STORE_BF16>(a, tiles, stream);
        case EPI_STORE_F32: return launch_one<C, GROUPED, EPI_STORE_F32>(a, tiles, stream);
        case EPI_ATOMIC_F32:
            if constexpr (!GROUPED) return launch_one<C, false, EPI_ATOMIC_F32>(a, tiles, stream);
            break;
        case EPI_OWNER_F32:
            if constexpr (!GROUPED) return launch_one<C, false, EPI_OWNER_F32>(a, tiles, stream);
            break;
    }
    return hipErrorInvalidValue;
}

template <bool GROUPED>
static hipError_t launch_cfg(const GemmArgs& a, TileCfgId cfg, Epi epi, int64_t tiles,
                             hipStream_t stream) {
    switch (cfg) {
        case CFG_256x256: return launch_epi<Cfg256x256, GROUPED>(a, epi, tiles, stream);
        case CFG_256x128: return launch_epi<Cfg256x128, GROUPED>(a, epi, tiles, stream);
        case CFG_256x128_2WG: return launch_epi<Cfg256x128x2, GROUPED>(a, epi, tiles, stream);
        case CFG_128x128: return launch_epi<Cfg128x128, GROUPED>(a, epi, tiles, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm(const GemmArgs& a, TileCfgId cfg, Epi epi, hipStream_t stream) {
    const TileShape t = tile_shape(cfg);
    const int64_t tiles = ((a.M + t.bm - 1) / t.bm) * ((a.N + t.bn - 1) / t.bn);
    return launch_cfg<false>(a, cfg, epi, tiles, stream);
}

hipError_t launch_grouped(const GemmArgs& a, TileCfgId cfg, Epi epi, int64_t max_tiles,
                          hipStream_t stream) {
    return launch_cfg<true>(a, cfg, epi, max_tiles, stream);
}

}  // namespace pk
