// bsp_attn.hip -- causal block-sparse prefill attention with dynamic block
// skipping inside the online softmax, for MI355X (gfx950, CDNA4).
//
// Method: page "长上下文推理加速方案部署实战：基于动态稀疏注意力机制的推理服务优化指南"
// (deployment guide for a dynamic sparse attention kernel), section 3.2 and
// section 6.1. For each (query tile, key block) pair the kernel computes the
// block's scores, each row's local maximum, compares it with the running
// maximum, and when every row's gap exceeds lambda it skips the
// exponentials, the V-block load and the PV product.
//
// Kernel organisation (one workgroup = one query tile of one or two query
// heads that share a KV head):
//   * block_q/32 waves of 64 lanes per head; wave w owns 32 query rows.
//   * scores are computed transposed, S^T = K Q^T, with 32x32 MFMA tiles:
//     keys are the M dimension (read from LDS), queries the N dimension
//     (held in registers for the whole tile). In the 32x32 accumulator
//     layout lane l holds query (l % 32) and 16 keys, so every per-row
//     reduction is 16 values in-lane plus one exchange with lane l ^ 32
//     (v_permlane32_swap).
//   * O^T = V^T P^T reuses the score accumulators directly as the B operand:
//     the contraction index is permuted to match the accumulator layout, and
//     the V^T operand comes from row-major V in LDS through transposing reads
//     (ds_read_b64_tr_b16).
//   * with two heads per workgroup the waves of the two heads share the SIMDs
//     and alternate matrix and vector phases half a block apart (ping-pong).
//   * the tile-wide skip decision is a wave vote (__all) followed by an
//     LDS AND across the waves; V is loaded only for blocks some query head
//     of the workgroup keeps.
//   * work items are ordered heaviest tile first; when the KV head count is a
//     multiple of 8 all query heads of one KV head run on one XCD (workgroup
//     ids are dealt round-robin to the 8 XCDs), so its K/V stay in that
//     XCD's L2.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>
#include <vector>
#include <type_traits>

#include "bsp_attn.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct FwdParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;
    int64_t lse_sh;                 // elements between heads of lse (= total tokens)
    const int32_t *cu;              // cu_seqlens
    const int32_t *table;           // paged: block table, else NULL
    int32_t max_pages;
    int32_t page_shift;             // log2(page_size)
    uint32_t *bitmap;               // NULL: not written
    unsigned long long *skip_count;
    unsigned long long *visited_count;
    int32_t n_seqs, T_max, W;       // W: bitmap words per (head, seq, tile) row
    int32_t Hq, Hkv, G;
    int32_t xcd_mode;               // 1: KV heads partitioned over the 8 XCDs
    int32_t hpw;                    // query heads per workgroup (divides G)
    float c_log2;                   // softmax scale * log2(e)
    float lam_raw;                  // lambda in raw dot-product units (lambda / scale)
    // fp8 inputs: per-head dequantisation scales (device, float); the kernel folds
    // q_scale[h] * k_scale[g] into its score scale and v_scale[g] into the output.
    const float *q_scale, *k_scale, *v_scale;
    float scale;                    // 1 / sqrt(head_dim)
    float lam;                      // lambda in natural-log units (+inf: dense)
    // chunked prefill: key/value bounds per sequence (NULL: same as cu); the
    // queries of a sequence are its last Lq of Lk positions
    const int32_t *cu_k;
    const float *lam_seq;           // lambda per sequence, or NULL
    unsigned long long *seq_skip, *seq_visited;  // counts per sequence, or NULL
    uint32_t flags;                 // BSP_FLAG_* ablation switches
    // dense mode run with other blocks than the caller's (results do not depend on
    // them at lambda = +inf): visited counts in the caller's (block_q, block_k); 0: the kernel's
    int32_t acct_bq, acct_bk;
    // sparse mode at block_q = 64 run on a 128-row tile: each 64-row half of the
    // tile takes its own decisions (the caller's tiles), 0: one decision per tile
    int32_t half_vote;
    int32_t T_bm;                   // bitmap tiles per (head, sequence) row: the caller's block_q
};

constexpr float kLn2 = 0.69314718055994530942f;

// Field of the kernel's single by-value argument (at offset 0 of the kernel
// argument segment), loaded where it is used: a volatile load that the compiler
// cannot hoist to the kernel entry, so the value does not hold a scalar register
// through the main loop. (Taking the address of the argument instead would make
// the compiler copy it to private memory.)
template <typename T>
__device__ __forceinline__ T late_kernel_arg(size_t offset) {
    const auto *seg = (const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr();
    return *(const volatile __attribute__((address_space(4))) T *)(seg + offset);
}
#define BSP_LATE_ARG(S, field) late_kernel_arg<decltype(S::field)>(offsetof(S, field))

#define BSP_LDS(T, ptr) ((__attribute__((address_space(3))) T *)(ptr))

// Map the workgroup id to (sequence, query tile, head group of HPW query heads
// that share one KV head). Tiles are dealt from the last (heaviest under the
// causal mask) to the first; in XCD mode the head groups of KV head x + 8i
// all run on XCD x.
__device__ __forceinline__ void decode_item(const FwdParams &p, int &s, int &t, int &hp) {
    const int b = blockIdx.x;
    const int Gp = p.G / p.hpw;          // head groups per KV head
    if (p.xcd_mode) {
        const int x = b & 7;
        const int slot = b >> 3;
        const int gpx = p.Hkv >> 3;      // KV heads per XCD
        const int per_tile = gpx * p.n_seqs * Gp;
        const int tr = slot / per_tile;
        int rem = slot - tr * per_tile;
        const int gi = rem / (p.n_seqs * Gp);
        rem -= gi * p.n_seqs * Gp;
        s = rem / Gp;
        const int e = rem - s * Gp;
        hp = (x + 8 * gi) * Gp + e;
        t = p.T_max - 1 - tr;
    } else {
        const int Hp = p.Hq / p.hpw;
        const int per_tile = p.n_seqs * Hp;
        const int tr = b / per_tile;
        const int rem = b - tr * per_tile;
        s = rem / Hp;
        hp = rem - s * Hp;
        t = p.T_max - 1 - tr;
    }
}

// Element offset of key/value row `kk` (sequence-local) of sequence s.
template <bool PAGED>
__device__ __forceinline__ int64_t kv_row(const FwdParams &p, int s, int base, int kk, int64_t st) {
    if constexpr (PAGED) {
        const int pg = p.table[(int64_t)s * p.max_pages + min(kk >> p.page_shift, p.max_pages - 1)];
        const int64_t slot = ((int64_t)pg << p.page_shift) + (kk & ((1 << p.page_shift) - 1));
        return slot * st;
    } else {
        return (int64_t)(base + kk) * st;
    }
}

// Maximum of the 16 values with m folded in, as a chain of three-operand
// maxima (v_max3_f32; the device code is built without NaN operands, so the
// compiler needs no operand canonicalisation).
__device__ __forceinline__ float max_fold16(float m, const f32x16 &a) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) m = fmaxf(fmaxf(m, a[i]), a[i + 1]);
    return m;
}
__device__ __forceinline__ float wave_max16(const f32x16 &a) { return max_fold16(-INFINITY, a); }

// Combine lanes l and l ^ 32 on the vector ALU: v_permlane32_swap of x with
// itself yields [x_lo, x_lo] and [x_hi, x_hi] (lanes 0-31 and 32-63), so
// every lane sees both halves without a round trip through LDS (ds_bpermute).
// The sum is x_lo + x_hi on every lane, equal to x + x[l ^ 32] in either order.
__device__ __forceinline__ void lane_halves(float x, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_max(float x) {
    float a, b;
    lane_halves(x, a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
    float a, b;
    lane_halves(x, a, b);
    return a + b;
}

// Keeps the scheduler from moving any instruction across this point: the
// interleaving written in the source (matrix, vector and copy instructions of
// independent work) is kept at that granularity.
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Shared epilogue of the decision: record the bit and the count.
struct SkipLog {
    uint32_t word = 0;
    int nskip = 0;
};

__device__ __forceinline__ void log_decision(const FwdParams &p, SkipLog &lg, int64_t row, int j, int nblk,
                                             bool skip, bool writer) {
    if (skip) {
        lg.word |= 1u << (j & 31);
        ++lg.nskip;
    }
    if ((j & 31) == 31 || j == nblk - 1) {
        // (j >> 5) < W unless the caller's max_seqlen(_k) understates a sequence: never write past the row
        if (p.bitmap != nullptr && writer && (j >> 5) < p.W) p.bitmap[row * p.W + (j >> 5)] = lg.word;
        lg.word = 0;
    }
}

// ---------------------------------------------------------------------------
// MFMA kernel for bf16 and fp8 e4m3 inputs, fp32 accumulation.
//
//   bf16: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16.
//   fp8 : S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x e4m3, per-head
//         dequantisation scales folded into the score scale); V is widened
//         from e4m3 to bf16 (exact) once per block in LDS and O^T = V^T P^T
//         runs on the bf16 MFMA with bf16 probabilities. Probabilities rounded
//         to e4m3 (3 mantissa bits) would cost up to ~6% of the dominant
//         term of a peaked row, too coarse for the output tolerance.
//
// A workgroup serves one query tile of HPW query heads that share a KV head
// (GQA grouping), with block_q/32 waves per head; K and V blocks are staged
// once in LDS for all of them. K and V move from global memory straight into
// LDS (global_load_lds, 16 bytes per lane), double-buffered, in row-major
// [key][dim] order with the 16-byte chunks of each row XOR-swizzled so that
// both the QK^T operand reads (ds_read_b128 along dim) and the transposing
// PV operand reads (ds_read_b64_tr_b16, which hands each lane four keys of one
// dim) are free of bank conflicts.
//
// Per key block j (software-pipelined: the PV product of a kept block runs one
// block later, next to the following block's softmax):
//   1. S^T = K_j Q^T, with the copy instructions of K_{j+1} spread over its
//      MFMAs; causal mask on the diagonal block; row maxima; per-head vote;
//      (fp8: widen the staged V_{j-1} into the bf16 V buffer); barrier B1
//      (which also publishes V_{j-1});
//   2. start the copy of V_j (bf16: into its buffer; fp8: into the staging
//      buffer) only if some head keeps block j;
//   3. softmax of block j (if kept) and O^T += V^T P^T of the previous kept
//      block from the V buffer; barrier B2 publishes K_{j+1}.
// Dense mode (lambda = +inf) is a kernel of its own: every block is kept, there
// is no vote, and step 3 interleaves each PV MFMA with a share of the
// exponentials and the row sum (fixed by scheduling fences), so that matrix
// cores and vector ALU overlap. The sparse kernel keeps step 3 unfused: the
// skip branches and the fused order together do not fit in the registers.
// The exponent reference max moves only when the running max has grown by
// more than 2^8 (base-2 units), so the O/l rescale is rare, except on the
// blocks the causal mask cuts, where it follows the running max exactly; the
// running max used by the skip decision is tracked exactly and separately.
// ---------------------------------------------------------------------------
constexpr float kRescaleLog2 = 8.0f;
// LDS operand reads in flight ahead of the MFMA that uses them (dense ping-pong matrix phase).
constexpr int kPingPongDepth = 6;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// XOR swizzle of the 16-byte chunks of a bf16 LDS row r (row = one key, 2*D bytes).
// D = 128 (one row per 256-byte bank window): rows 0..15 get sixteen distinct
// XORs (conflict-free ds_read_b128 of one chunk over 16 rows), and the four
// rows that one half-wave of a transposing PV read touches (r, r+1, r+2, r+3 for
// r % 4 == 0) land their four 16-byte chunks in four distinct 64-byte groups.
template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return 2 * ((r >> 1) & 3);
}

// XOR swizzle of the 16-byte chunks of an fp8 K row r (128 bytes: two rows per
// 256-byte bank window). The eight rows of equal parity among sixteen
// consecutive rows get eight distinct chunk XORs, so the sixteen lanes that
// one ds_read_b128 cycle serves (rows 0..15 of a tile, one logical chunk) hit
// sixteen distinct 16-byte bank groups.
__device__ __forceinline__ int chunk_swz8(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16-byte global -> LDS copy for the whole wave: lane l's 16 bytes from `gptr`
// land at LDS byte address lds + 16 l (lds must be wave-uniform). Issued from
// inline assembly so that the compiler does not serialise it against unrelated
// LDS reads; completion is awaited explicitly (s_waitcnt vmcnt) before the
// barrier that publishes the buffer.
__device__ __forceinline__ void lds_copy16(const void *gptr, const void *lds) {
    const uint32_t la = (uint32_t)(uintptr_t)BSP_LDS(const void, lds);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(la) : "m0");
}
// Same copy with a wave-uniform 64-bit base (SGPR pair) and a per-lane 32-bit
// byte offset: the per-copy address arithmetic stays on the scalar unit.
__device__ __forceinline__ void lds_copy16_sb(const void *sbase, uint32_t voff, const void *lds) {
    const uint32_t la = (uint32_t)(uintptr_t)BSP_LDS(const void, lds);
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(la) : "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmem_leave() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Two e4m3 codes (bytes 2*HI and 2*HI+1 of x) widened to bf16; exact, since
// every e4m3 value (subnormals included) is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x) {
    const bf16x2 y = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, y);
}

// KH: sparse mode for a caller's 64-key blocks on 128-key blocks. Each 64-key
// half of a block is decided on its own, in key order, and under half-tile votes
// (FwdParams::half_vote) each 64-row half of the tile as well.
template <int IN, int D, int BQ, int BK, bool PAGED, int HPW, bool DENSE, bool KH = false>
__global__ void __launch_bounds__(BQ * 2 * HPW, (BQ == 64 && HPW == 2) ? 2 : 1) fwd_mfma(FwdParams p) {
    constexpr bool F8 = IN == BSP_FP8_E4M3;
    constexpr int WPH = BQ / 32;     // waves per head
    constexpr int NW = WPH * HPW;    // waves per workgroup
    constexpr int ES = F8 ? 1 : 2;   // bytes per input element
    constexpr int KS = F8 ? D / 64 : D / 16;  // k-steps of S^T = K Q^T
    constexpr int MT = BK / 32;      // 32-key tiles of a block
    constexpr int DT = D / 32;       // 32-dim tiles of O^T
    constexpr int PC = BK / 16;      // 16-key chunks of the PV contraction
    constexpr int KROWB = D * ES;    // bytes per LDS row of K (and of the fp8 V staging buffer)
    constexpr int KCPR = KROWB / 16; // 16-byte chunks per such row
    constexpr int KBLKB = BK * KROWB;
    constexpr int KRPK = 1024 / KROWB;  // rows per 1 KB wave copy
    constexpr int CI = KBLKB / 1024 / NW;  // copy instructions per wave per block
    constexpr int VROWB = D * 2;     // bytes per LDS row of V (bf16 for both input types)
    constexpr int VBLKB = BK * VROWB;
    // Ping-pong dense schedule: two query heads of four waves each, so that waves
    // w and w + 4 (which share a SIMD) belong to different heads.
    // Sparse mode runs the same schedule with a vote after QK (SPP), except the
    // fp8 paged instance, which would not fit the registers.
    constexpr bool PP = DENSE && HPW == 2 && WPH == 4;
    constexpr bool SPP = !DENSE && HPW == 2 && WPH == 4 && !(F8 && PAGED);
    // bf16 V buffers (the lockstep fp8 loop widens V in a phase of its own and needs one)
    constexpr int NVB = (F8 && !PP && !SPP) ? 1 : 2;
    static_assert(KBLKB % (1024 * NW) == 0, "block copy must split evenly over the waves");
    static_assert(!KH || (SPP && BK == 128), "key-half votes run on the two-head sparse schedule at 128-key blocks");
    static_assert(!F8 || D == 128, "fp8 kernels are built for head_dim 128");
    __shared__ __attribute__((aligned(1024))) char sK[2][KBLKB];
    __shared__ __attribute__((aligned(1024))) char sV[NVB][VBLKB];
    // fp8 V staging; the sparse two-head schedule can have the copies of two blocks in flight
    constexpr int NV8 = (F8 && SPP) ? 2 : 1;
    __shared__ __attribute__((aligned(1024))) char sV8[NV8][F8 ? KBLKB : 16];
    __shared__ __attribute__((aligned(16))) int sVote[NW];
    __shared__ int sHead;  // two-head sparse schedule: 1 if head 0 keeps the block it decided last

    int s, t, hp;
    decode_item(p, s, t, hp);  // hp: index of the head group served by this workgroup
    const int base = p.cu[s];
    const int L = p.cu[s + 1] - base;  // query rows of the sequence (its chunk)
    if (t * BQ >= L) return;  // tile past the end of this sequence (bitmap row stays zero)
    const int kbase = p.cu_k ? p.cu_k[s] : base;
    const int Lk = p.cu_k ? p.cu_k[s + 1] - kbase : L;  // keys of the sequence
    const int off = Lk - L;            // query row r sits at key position off + r
    if (off < 0) return;               // a chunk longer than its sequence: caller error, nothing written

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform: keeps wave data in SGPRs)
    const int hl = w / WPH;            // head of this wave within the workgroup
    const int wq = w - hl * WPH;       // wave index within its head
    const int h = hp * HPW + hl;
    const int ln = lane & 31;
    const int hh = lane >> 5;
    const int g = h / p.G;
    const int r1 = min((t + 1) * BQ, L);
    const int nblk = (off + r1 - 1) / BK + 1;  // causal: up to the block of key position off + r1 - 1
    const int q0 = t * BQ + wq * 32;
    const int qrow = q0 + ln;
    const bool valid = qrow < L;
    const int qpos = off + qrow;       // key position of this lane's query
    constexpr bool dense = DENSE;  // lambda = +inf: every block is kept, no vote
    // Decisions this wave records on the two-head sparse schedule: nlog blocks of
    // bitmap tile tb (0 for a wave that records nothing). One tile-wide decision:
    // wave 0 of each head records all visited blocks of the tile. Half-tile votes
    // (the caller's block_q is 64): waves 0 and 2 record the causal blocks of
    // their 64-row half, tile 2t or 2t + 1 in the caller's units.
    // Key-half votes (the caller's block_k is 64): nlog counts the caller's blocks.
    int tb = t, nlog = nblk;
    if constexpr (SPP) {
        constexpr int cbk = KH ? BK / 2 : BK;
        if (KH && p.half_vote != 0) {
            tb = 2 * t + (wq >> 1);
            const int r0 = tb * (BQ / 2);
            nlog = ((wq & 1) == 0 && r0 < L) ? (off + min(r0 + BQ / 2, L) - 1) / cbk + 1 : 0;
        } else {
            nlog = wq == 0 ? (off + r1 - 1) / cbk + 1 : 0;
        }
    }
    const int64_t bm_row = ((int64_t)h * p.n_seqs + s) * p.T_bm + tb;
    float c = p.c_log2;           // raw score -> base-2 exponent
    float lam_raw = p.lam_raw;    // lambda in raw score units
    float osc = 1.f;              // output scale
    float sqk = 1.f;
    if constexpr (F8) {
        sqk = p.q_scale[h] * p.k_scale[g];
        c = p.c_log2 * sqk;
        if (!dense) lam_raw = p.lam / (p.scale * sqk);
        osc = p.v_scale[g];
    }
    if (!dense && p.lam_seq != nullptr) {
        const float ls = p.lam_seq[s];
        lam_raw = ls == INFINITY ? INFINITY : ls / (p.scale * sqk);
    }

    const char *kg = (const char *)p.k + (int64_t)g * p.k_sh * ES;
    const char *vg = (const char *)p.v + (int64_t)g * p.v_sh * ES;
    const int64_t kstb = p.k_st * ES;  // bytes between tokens
    const int64_t vstb = p.v_st * ES;

    // Q^T fragments (MFMA B operand). bf16: lane holds Q[qrow][16ks + 8hh .. +7];
    // fp8: lane holds Q[qrow][64ks + 32hh .. +31]. The K operand reads below use
    // the same dims per (lane half, byte), so the contraction pairs like with like.
    typedef typename std::conditional<F8, i32x8, bf16x8>::type QFrag;
    QFrag qf[KS];
    {
        const char *qp = (const char *)p.q + ((int64_t)(base + (valid ? qrow : 0)) * p.q_st + (int64_t)h * p.q_sh) * ES;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if constexpr (F8) {
                const u32x4 lo = *(const u32x4 *)(qp + 64 * ks + 32 * hh);
                const u32x4 hi = *(const u32x4 *)(qp + 64 * ks + 32 * hh + 16);
                i32x8 x = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                if (!valid) x = i32x8{};
                qf[ks] = x;
            } else {
                bf16x8 x = *(const bf16x8 *)(qp + 2 * (16 * ks + 8 * hh));
                if (!valid) x = bf16x8{};
                qf[ks] = x;
            }
        }
    }

    // Copy of the key/value block starting at key kb into an LDS buffer. Wave
    // w's i-th copy instruction fills the 1 KB segment i*NW + w; lane l writes
    // physical chunk l % KCPR of row crow0 + i*CSTEP and fetches the logical
    // chunk that the swizzle maps there (fp8 V staging: no swizzle). When CSTEP
    // is a multiple of the swizzle period (16 rows) that chunk is the same for
    // every copy of the lane. Rows past the sequence end re-read its last row
    // (finite data, always masked; the K copy one block past the last one of a
    // tile is of this kind). Each copy instruction is issued on its own, so
    // that the copies of a block can be spread over the matrix work. The code is
    // branch-free: packed K/V use a wave-uniform base at row kb0 = min(kb, L-1)
    // and a per-lane 32-bit offset (kk - kb0) * stride + chunk, which lies in
    // [0, (BK - 1) * stride + 16 * (KCPR - 1)] because kb0 <= kk <= L - 1.
    auto kswz = [](int r) -> int {
        if constexpr (F8) return chunk_swz8(r);
        else return chunk_swz<D>(r);
    };
    constexpr int CSTEP = NW * KRPK;
    constexpr bool kFixedChunk = CSTEP % 16 == 0;
    constexpr int kLog2Rpk = KRPK == 8 ? 3 : KRPK == 4 ? 2 : KRPK == 2 ? 1 : 0;
    static_assert((1 << kLog2Rpk) == KRPK, "rows per copy must be a power of two");
    const int crow0 = w * KRPK + lane / KCPR;
    const int lcK = 16 * ((lane % KCPR) ^ kswz(crow0));
    // dw: copy the share of wave w + dw instead of this wave's (the two-head sparse schedule lets
    // the waves of one head copy a whole V block); |dw| * KRPK is a multiple of the swizzle period.
    auto copy_one = [&](const char *src, int64_t stb, int kb, char *dst, bool swz, int i, int dw = 0) {
        const int o = i * CSTEP + dw * KRPK;  // row offset of this copy from row crow0
        const int r = crow0 + o;
        const int kk = min(kb + r, Lk - 1);
        const int lci = !swz ? 16 * (lane % KCPR) : kFixedChunk ? lcK : 16 * ((lane % KCPR) ^ kswz(r));
        if constexpr (PAGED) {
            // (more than 4 copies per wave hold too many page bases in scalar registers)
            if (CI <= 4 && p.page_shift >= kLog2Rpk) {
                // The instruction's KRPK rows (KRPK-aligned) lie in one page, also after
                // clamping, so the page id is wave-uniform: a scalar load, which does
                // not wait behind the copies in flight as a vector load would.
                const int r0 = __builtin_amdgcn_readfirstlane(min(kb + w * KRPK + o, Lk - 1));
                // read-only table through the constant address space: a uniform index
                // becomes s_load_dword
                const auto *tbl = (const __attribute__((address_space(4))) int32_t *)p.table;
                const int pg = __builtin_amdgcn_readfirstlane(
                    tbl[(int64_t)s * p.max_pages + min(r0 >> p.page_shift, p.max_pages - 1)]);
                const char *pbase = src + ((int64_t)pg << p.page_shift) * stb;
                lds_copy16_sb(pbase, (uint32_t)((kk & ((1 << p.page_shift) - 1)) * stb) + (uint32_t)lci,
                              dst + (i * NW + w + dw) * 1024);
            } else {
                lds_copy16(src + kv_row<PAGED>(p, s, kbase, kk, stb) + lci, dst + (i * NW + w + dw) * 1024);
            }
        } else {
            // row kk - kb0 = min(r, lim) with lim = min(Lk - 1 - kb0, BK - 1), as
            // min(crow0, lim - o) * stride + o * stride: one vector min and one add per
            // copy (the per-lane crow0 * stride is loop-invariant); every term is below
            // BK * stride < 2^31.
            const int kb0 = min(kb, Lk - 1);
            const int sb = (int)stb;
            const int lim = min(Lk - 1 - kb0, BK - 1);
            const int rowb = min(crow0 * sb, (lim - o) * sb) + o * sb + lci;
            lds_copy16_sb(src + (int64_t)(kbase + kb0) * stb, (uint32_t)rowb, dst + (i * NW + w + dw) * 1024);
        }
    };
    auto copy_block = [&](const char *src, int64_t stb, int kb, char *dst, bool swz) {
#pragma unroll
        for (int i = 0; i < CI; ++i) copy_one(src, stb, kb, dst, swz, i);
    };
    // fp8: widen this wave's own staged V bytes (its copies of the block, landed
    // once vmcnt says so) into the bf16 V buffer, in the bf16 row swizzle.
    auto widen_v = [&](char *vdst, int stage = 0, int dw = 0) {
        if constexpr (F8) {
#pragma unroll
            for (int i = 0; i < CI; ++i) {
                const int r = crow0 + i * CSTEP + dw * KRPK;
                const int c16 = lane % KCPR;
                const u32x4 x = *(const u32x4 *)(sV8[stage] + (i * NW + w + dw) * 1024 + 16 * lane);
                const u32x4 lo = {fp8x2_to_bf16x2<false>(x[0]), fp8x2_to_bf16x2<true>(x[0]),
                                  fp8x2_to_bf16x2<false>(x[1]), fp8x2_to_bf16x2<true>(x[1])};
                const u32x4 hi = {fp8x2_to_bf16x2<false>(x[2]), fp8x2_to_bf16x2<true>(x[2]),
                                  fp8x2_to_bf16x2<false>(x[3]), fp8x2_to_bf16x2<true>(x[3])};
                char *row = vdst + r * VROWB;
                *(u32x4 *)(row + (((2 * c16) ^ chunk_swz<D>(r)) << 4)) = lo;
                *(u32x4 *)(row + (((2 * c16 + 1) ^ chunk_swz<D>(r)) << 4)) = hi;
            }
        }
    };

    float m_dec = -INFINITY;  // running max of raw scores <q,k> (skip decision)
    float m_ref = -INFINITY;  // reference max of the exponentials (lags m_dec by < 2^8 in base 2)
    float l_run = 0.f;
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
    SkipLog lg;

    // K operand reads: row 32mt + ln (the swizzle repeats every 16 rows, so it is that of row ln).
    const int krow = ln * KROWB;
    const int ksw = kswz(ln);

    // PV operand reads: contraction chunk cc = 2mt + u covers keys 32mt + 16u + 8(i'/4) + 4hh + i'%4
    // (i' = 0..7). Two transposing reads give lane (dim d, half hh) those 8 keys: in each 16-lane
    // group, source lane i points at key 32mt + 16u + 4hh + i/4 (+8), dims d0 + 4(i%4)..+3. The
    // swizzle depends on the key only through key % 16, so the offset of chunk cc is that of
    // chunk 0 plus the immediate cc * 16 * VROWB; the second read (keys +8) differs only in
    // swizzle bit 1 (D = 128: chunk offset ^ 32 bytes) or not at all (D = 64).
    int vrd_off[DT];
    {
        const int grp = lane >> 4;
        const int gi = lane & 15;
        const int dsub = 16 * (grp & 1) + 4 * (gi & 3);
        const int r0 = 4 * (grp >> 1) + (gi >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int d = 32 * dt + dsub;
            vrd_off[dt] = r0 * VROWB + (((d >> 3) ^ chunk_swz<D>(r0)) << 4) + (d & 7) * 2;
        }
    }
    auto vread_at = [&](const char *vbuf, int cc, int dt) -> bf16x8 {
        const int o0 = vrd_off[dt] + cc * 16 * VROWB;
        const int o8 = (D == 128 ? (vrd_off[dt] ^ 32) : vrd_off[dt]) + cc * 16 * VROWB + 8 * VROWB;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(BSP_LDS(bf16x4, vbuf + o0));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(BSP_LDS(bf16x4, vbuf + o8));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    // O^T += V^T P^T for a kept block whose bf16 probabilities are in pp and whose V is in vbuf.
    auto pv_block = [&](const bf16x8 *pp, const char *vbuf) {
#pragma unroll
        for (int cc = 0; cc < PC; ++cc) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread_at(vbuf, cc, dt), pp[cc], oacc[dt], 0, 0, 0);
        }
    };

    copy_block(kg, kstb, 0, sK[0], true);
    wait_vmem_all();
    __syncthreads();

    bf16x8 pprev[PC];       // probabilities of this wave's last kept block, PV still pending
    bool pend = false;      // wave-uniform: a PV is pending
    bool v_prev = false;    // workgroup-uniform: V of block j-1 was copied
    constexpr int NE = 16 * MT;        // scores per lane per block
    constexpr int NPV = PC * DT;       // MFMAs of the PV product
    constexpr int EPG = NE / NPV;      // exponentials per PV MFMA
    static_assert(NE % NPV == 0, "softmax/PV interleave must be even");
    f32x16 sacc[MT];
    float pe[NE];           // probabilities of the current block, element e = 16 mt + i

    // Causal mask of the block at key kb (called only where the block reaches
    // past this wave's first query): key 32mt + 8(i/4) + 4hh + i%4 of the block
    // is hidden from query position qpos iff 32mt + 8(i/4) + i%4 > qpos - kb - 4hh.
    // One compare and select per element, fenced, so that a single lane mask is
    // live at a time (all 64 masks at once exhaust the scalar registers).
    auto causal_mask = [&](int kb) {
        const int d = qpos - kb - 4 * hh;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sacc[mt][i] = (32 * mt + 8 * (i >> 2) + (i & 3) > d) ? -INFINITY : sacc[mt][i];
                SCHED_FENCE();
            }
    };

    // ---- S^T = K_j Q^T : sacc[mt] holds keys 32mt + 8(i/4) + 4hh + i%4 for query qrow;
    // causal mask; returns the row maximum over the block. MFMA f = ks*MT + mt
    // (k-step outermost, so consecutive MFMAs use independent accumulators); its K
    // operand is read one MFMA ahead, and the copy instructions of K_{j+1} are
    // spread over the MFMAs (one every QSTEP), which keeps them from queueing at
    // the memory unit all at once.
    auto qk_phase = [&](int j) -> float {
        const int kb = j * BK;
        const char *kbuf = sK[j & 1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sacc[mt] = f32x16{};
        constexpr int NQK = KS * MT;
        constexpr int QSTEP = NQK / CI;
        static_assert(NQK % CI == 0, "K copies must spread evenly over the QK MFMAs");
        typedef typename std::conditional<F8, i32x8, bf16x8>::type KOp;
        auto kread = [&](int f) -> KOp {
            const int ks = f / MT, mt = f % MT;
            const char *rowp = kbuf + krow + 32 * mt * KROWB;
            if constexpr (F8) {
                const u32x4 lo = *(const u32x4 *)(rowp + (((4 * ks + 2 * hh) ^ ksw) << 4));
                const u32x4 hi = *(const u32x4 *)(rowp + (((4 * ks + 2 * hh + 1) ^ ksw) << 4));
                return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            } else {
                return *(const bf16x8 *)(rowp + (((2 * ks + hh) ^ ksw) << 4));
            }
        };
        KOp kop[NQK];
        kop[0] = kread(0);
#pragma unroll
        for (int f = 0; f < NQK; ++f) {
            if (f + 1 < NQK) kop[f + 1] = kread(f + 1);
            const int ks = f / MT, mt = f % MT;
            if constexpr (F8) sacc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[f], qf[ks], sacc[mt], 0, 0, 0, 0, 0, 0);
            else sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[f], qf[ks], sacc[mt], 0, 0, 0);
            if (f % QSTEP == 0) {  // K_{j+1} (rows clamped: past the last block it re-reads the end)
                SCHED_FENCE();
                copy_one(kg, kstb, kb + BK, sK[(j + 1) & 1], true, f / QSTEP);
                SCHED_FENCE();
            }
        }
        if (kb + BK - 1 > off + q0) causal_mask(kb);
        float m = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) m = max_fold16(m, sacc[mt]);
        return halves_max(m);
    };

    // Running max, lazy reference update; returns (in mc) the reference in
    // base-2 units, and the rescale factor for O and l (resc: needed by a lane).
    // On the blocks the causal mask cuts (those holding the tile's own keys) the
    // reference follows every growth of the running max, so that a row whose
    // weight sits on a nearby key gets probability exactly 1 there: a lagging
    // reference would give it 2^d with d in (0, 8], which the bf16 rounding of P
    // perturbs by up to 2^-9 of that key's whole contribution. At most one extra
    // rescale per tile.
    auto new_reference = [&](float mloc, int kb, float &alpha, bool &resc) -> float {
        const float m_new = fmaxf(m_dec, mloc);
        m_dec = m_new;
        const float lag = kb + BK - 1 > off + q0 ? 0.f : kRescaleLog2;
        const bool need = (m_new - m_ref) * c > lag;  // also true while m_ref = -inf
        resc = __any(need);
        alpha = 1.f;
        if (need) {
            alpha = (m_ref == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_new) * c);
            m_ref = m_new;
        }
        return m_ref * c;
    };
    // O and l to the new reference (after the pending PV), l += row sum, and the
    // bf16 probabilities of this block for its PV product.
    auto finish_block = [&](float rs, float alpha, bool resc) {
        rs = halves_sum(rs);
        if (resc) {
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        }
        l_run += rs;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) pprev[2 * mt + u][i] = (__bf16)pe[16 * mt + 8 * u + i];
    };
    auto exp_sum = [&](float mc) -> float {
        float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], c, -mc));
#pragma unroll
        for (int e = 0; e < NE; e += 2) {
            rs0 += pe[e];
            rs1 += pe[e + 1];
        }
        return rs0 + rs1;
    };

    // PV of the previous kept block (V in vbuf) interleaved with the exponentials
    // and row sum of the current block: group g is PV MFMA g (V operand read one
    // MFMA ahead) followed by the exponentials of elements EPG*g .. EPG*g + EPG - 1
    // and the row sum of the previous group's elements, so the matrix cores and
    // the vector ALU work side by side. The fences keep this order. Returns the
    // row sum (this lane's half).
    auto fused_pv_exp = [&](const char *vbuf, float mc) -> float {
        auto vread = [&](int g) -> bf16x8 { return vread_at(vbuf, g / DT, g % DT); };
        float rs0 = 0.f, rs1 = 0.f;
        bf16x8 vop[NPV];
        vop[0] = vread(0);
#pragma unroll
        for (int g = 0; g < NPV; ++g) {
            if (g + 1 < NPV) vop[g + 1] = vread(g + 1);
            oacc[g % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[g], pprev[g / DT], oacc[g % DT], 0, 0, 0);
#pragma unroll
            for (int e = EPG * g; e < EPG * (g + 1); ++e)
                pe[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], c, -mc));
            if (g > 0) {
#pragma unroll
                for (int e = EPG * (g - 1); e < EPG * g; e += 2) {
                    rs0 += pe[e];
                    rs1 += pe[e + 1];
                }
            }
            SCHED_FENCE();
        }
#pragma unroll
        for (int e = NE - EPG; e < NE; e += 2) {
            rs0 += pe[e];
            rs1 += pe[e + 1];
        }
        return rs0 + rs1;
    };


    if constexpr (PP || SPP) {
        // ---- ping-pong. Per block j every wave runs a matrix phase
        // M_j = PV_{j-1} + QK_j and a vector phase V_j (mask, max, reference,
        // exponentials, row sum, bf16 probabilities). Head 1 runs half a block
        // behind head 0, the two separated by workgroup barriers: while head 0
        // runs M_j head 1 runs V_{j-1}, and while head 0 runs V_j head 1 runs
        // M_j. Each SIMD then holds one wave in a matrix phase and one in a
        // vector phase at all times, and its matrix cores and vector ALU work
        // side by side instead of taking turns. Interval 2j is the one in
        // which head 0 runs M_j; at its start every wave issues its share of
        // the copies of K_{j+1} and V_j. Each wave waits for its copies at the
        // end of interval 2j + 1, so they have two intervals to land, and they
        // fill the buffers of K_{j-1} and V_{j-2}, whose last reader (head 1's
        // M_{j-1}) ran in interval 2j - 1.
        auto issue_copy = [&](int j, int i) {  // copy i of this wave's share (K first, then V)
            if (i < CI) copy_one(kg, kstb, (j + 1) * BK, sK[(j + 1) & 1], true, i);
            else if constexpr (F8) copy_one(vg, vstb, j * BK, sV8[j & (NV8 - 1)], false, i - CI);  // fp8 V: staged, widened later
            else copy_one(vg, vstb, j * BK, sV[j & 1], true, i - CI);
        };
        // fp8: once its copies of V_j have landed, each wave widens them into the bf16 buffer of block j
        auto land_v = [&](int j) {
            if constexpr (F8) widen_v(sV[j & 1], j & (NV8 - 1));
        };
        // M phase: PV_{j-1} (probabilities pprev, V_{j-1} in LDS) and then QK_j
        // (K_j in LDS -> sacc). Only one wave of the SIMD issues matrix work in
        // this interval, so the LDS operand of MFMA s is read PD MFMAs ahead to
        // cover the read latency; running PV first and QK second keeps the
        // score accumulators dead while pprev is live. When this wave issues
        // the copies of the interval here, they go one every CSLOT MFMAs.
        auto m_phase = [&](int j, auto do_pv, auto do_qk, auto do_copy) {
            constexpr bool PV = decltype(do_pv)::value, QK = decltype(do_qk)::value;
            constexpr bool CP = decltype(do_copy)::value;
            constexpr int NQK = KS * MT;
            constexpr int P0 = PV ? NPV : 0;       // first QK slot
            constexpr int NS = P0 + (QK ? NQK : 0);
            constexpr int PD = kPingPongDepth;
            constexpr int CSLOT = NS / (2 * CI);
            static_assert(!CP || NS % (2 * CI) == 0, "copies must spread evenly over the matrix phase");
            const char *kbuf = sK[j & 1];
            const char *vbuf = sV[(j - 1) & 1];
            typedef typename std::conditional<F8, i32x8, bf16x8>::type KOp;
            bf16x8 vop[NS];  // V operands of the PV slots
            KOp kop[NS];     // K operands of the QK slots (fp8: 64 dims of a row per lane half)
            auto opread = [&](int x) {
                if (x < P0) {
                    vop[x] = vread_at(vbuf, x / DT, x % DT);
                } else {
                    const int f = x - P0, ks = f / MT, mt = f % MT;
                    const char *rowp = kbuf + krow + 32 * mt * KROWB;
                    if constexpr (F8) {
                        const u32x4 lo = *(const u32x4 *)(rowp + (((4 * ks + 2 * hh) ^ ksw) << 4));
                        const u32x4 hi = *(const u32x4 *)(rowp + (((4 * ks + 2 * hh + 1) ^ ksw) << 4));
                        kop[x] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    } else {
                        kop[x] = *(const bf16x8 *)(rowp + (((2 * ks + hh) ^ ksw) << 4));
                    }
                }
            };
            // This wave's MFMAs issue ahead of its SIMD partner's vector work.
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int x = 0; x < PD && x < NS; ++x) opread(x);
#pragma unroll
            for (int x = 0; x < NS; ++x) {
                if (x + PD < NS) opread(x + PD);
                if (x < P0) {
                    oacc[x % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[x], pprev[x / DT], oacc[x % DT], 0, 0, 0);
                } else {
                    const int f = x - P0;
                    const f32x16 c0 = f < MT ? f32x16{} : sacc[f % MT];
                    if constexpr (F8)
                        sacc[f % MT] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[x], qf[f / MT], c0, 0, 0, 0, 0, 0, 0);
                    else
                        sacc[f % MT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[x], qf[f / MT], c0, 0, 0, 0);
                }
                if constexpr (CP) {
                    if (x % CSLOT == 0) {
                        SCHED_FENCE();
                        issue_copy(j, x / CSLOT);
                    }
                }
                SCHED_FENCE();
            }
            __builtin_amdgcn_s_setprio(0);
        };
        // V phase of block j; the copies of the interval (when this wave issues
        // them here, for block cj) go one per group of exponentials.
        auto v_phase = [&](int j, auto do_copy, int cj) {
            constexpr bool CP = decltype(do_copy)::value;
            constexpr int EG = NE / (2 * CI);  // exponentials per copy
            const int kb = j * BK;
            if (kb + BK - 1 > off + q0) causal_mask(kb);
            float m = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) m = max_fold16(m, sacc[mt]);
            m = halves_max(m);
            float alpha;
            bool resc;
            const float mc = new_reference(m, kb, alpha, resc);
            float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                pe[e] = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], c, -mc));
                if (e & 1) {
                    rs0 += pe[e - 1];
                    rs1 += pe[e];
                }
                if constexpr (CP) {
                    if (e % EG == EG - 1) {
                        SCHED_FENCE();
                        issue_copy(cj, e / EG);
                        SCHED_FENCE();
                    }
                }
            }
            finish_block(rs0 + rs1, alpha, resc);
        };

        // ---- sparse mode on the same schedule. The matrix phase is split into a
        // PV part, run only if this head kept block j - 1, with its own operand
        // prologue (so the branch around it leaves one register assignment), and
        // a QK part that also carries the interval's K copies and ends with this
        // wave's vote on block j (causal mask, row max, every valid row's gap to
        // the running max above lambda). The barrier after the matrix phase
        // publishes the votes; the vector phase reads the head's votes (unless
        // this wave's own vote already keeps the block), records the decision,
        // and for a kept block runs the reference update,
        // exponentials and row sum. V_j is copied only after a head has decided
        // to keep block j (the V-load skip, below).
        float mloc_a = -INFINITY, mloc_b = -INFINITY;  // row maxima of the block's two key halves
        int my_vote = 0;  // wave-uniform: this wave's vote on its last QK block
        auto pv_part = [&](int j) {  // PV_{j-1}
            constexpr int PD = kPingPongDepth;
            const char *vbuf = sV[(j - 1) & 1];
            bf16x8 vop[NPV];
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int x = 0; x < PD && x < NPV; ++x) vop[x] = vread_at(vbuf, x / DT, x % DT);
#pragma unroll
            for (int x = 0; x < NPV; ++x) {
                if (x + PD < NPV) vop[x + PD] = vread_at(vbuf, (x + PD) / DT, (x + PD) % DT);
                oacc[x % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[x], pprev[x / DT], oacc[x % DT], 0, 0, 0);
                SCHED_FENCE();
            }
            __builtin_amdgcn_s_setprio(0);
        };
        // QK_j with copy slots spread over its MFMAs (one every CSLOT), vote. With NCP = 2 CI slots,
        // vmode (wave-uniform) picks the copies: bit 0 this wave's share of K_{j+1} (slots 0 .. CI-1),
        // bit 1 its share of V_j (slots CI .. 2CI-1, or 0 .. CI-1 when K is not copied).
        auto qk_vote = [&](int j, auto n_copies, int vmode = 3) {
            constexpr int NCP = decltype(n_copies)::value;
            constexpr bool CP = NCP > 0;
            constexpr int NQK = KS * MT;
            constexpr int PD = kPingPongDepth;
            constexpr int CSLOT = NQK / (CP ? NCP : 1);
            static_assert(!CP || NQK % NCP == 0, "copies must spread evenly over the QK MFMAs");
            const char *kbuf = sK[j & 1];
            typedef typename std::conditional<F8, i32x8, bf16x8>::type KOp;
            KOp kop[NQK];
            auto kread = [&](int f) {
                const int ks = f / MT, mt = f % MT;
                const char *rowp = kbuf + krow + 32 * mt * KROWB;
                if constexpr (F8) {
                    const u32x4 lo = *(const u32x4 *)(rowp + (((4 * ks + 2 * hh) ^ ksw) << 4));
                    const u32x4 hi = *(const u32x4 *)(rowp + (((4 * ks + 2 * hh + 1) ^ ksw) << 4));
                    kop[f] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                } else {
                    kop[f] = *(const bf16x8 *)(rowp + (((2 * ks + hh) ^ ksw) << 4));
                }
            };
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int f = 0; f < PD && f < NQK; ++f) kread(f);
#pragma unroll
            for (int f = 0; f < NQK; ++f) {
                if (f + PD < NQK) kread(f + PD);
                const f32x16 c0 = f < MT ? f32x16{} : sacc[f % MT];
                if constexpr (F8)
                    sacc[f % MT] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop[f], qf[f / MT], c0, 0, 0, 0, 0, 0, 0);
                else
                    sacc[f % MT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[f], qf[f / MT], c0, 0, 0, 0);
                if constexpr (CP) {
                    if (f % CSLOT == 0) {
                        SCHED_FENCE();
                        const int i = f / CSLOT;
                        if (i < CI) {
                            if (vmode & 1) issue_copy(j, i);
                            else if (vmode & 2) issue_copy(j, CI + i);
                        } else if ((vmode & 3) == 3) {
                            issue_copy(j, i);
                        }
                    }
                }
                SCHED_FENCE();
            }
            __builtin_amdgcn_s_setprio(0);
            const int kb = j * BK;
            if (kb + BK - 1 > off + q0) causal_mask(kb);
            // every valid row's gap from running max mr to block max ml exceeds lambda
            auto passes = [&](float mr, float ml) { return !valid || ml == -INFINITY || mr - ml > lam_raw; };
            int vote;
            if constexpr (KH) {
                // row maxima of the two key halves (keys 0..BK/2-1 sit in tiles mt < MT/2);
                // bit 0: first half; bits 1 and 2: second half if the first is skipped / kept
                float ma = -INFINITY, mb = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    if (mt < MT / 2) ma = max_fold16(ma, sacc[mt]);
                    else mb = max_fold16(mb, sacc[mt]);
                }
                mloc_a = halves_max(ma);
                mloc_b = halves_max(mb);
                vote = (__all(passes(m_dec, mloc_a)) ? 1 : 0) | (__all(passes(m_dec, mloc_b)) ? 2 : 0) |
                       (__all(passes(fmaxf(m_dec, mloc_a), mloc_b)) ? 4 : 0);
            } else {
                // one decision per block: its maximum stands in the first half's slot
                float m = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) m = max_fold16(m, sacc[mt]);
                mloc_a = halves_max(m);
                mloc_b = -INFINITY;
                vote = __all(passes(m_dec, mloc_a)) ? 1 : 0;
            }
            if (lane == 0) sVote[w] = vote;
            my_vote = vote;
        };
        // Vector phase of block j in sparse mode: the head's decision, then, for a
        // kept block, the reference update, exponentials (in place in the score
        // registers), row sum and bf16 probabilities. A skipped block zeroes the
        // probabilities instead, so that they are dead from a PV part to the next
        // vector phase on both paths (else they stay live through QK next to the
        // scores). The copies this wave issues in its vector phase go right after
        // the decision (after_vote(hk), hk = 1 if some wave of this head keeps
        // block j): before the decision they delay its vote read, interleaved
        // with the exponentials they cost the instance its registers.
        // Ablation (BSP_FLAG_EXP_SKIPPED): a skipped block's exponentials are
        // taken on the kept path against +inf (its maximum is left out of the
        // running max), so they come out zero and are dropped. Under key-half
        // votes a block whose halves are decided apart runs the kept path, the
        // skipped half's exponentials again taken against +inf.
        //
        // head_keeps(x): 1 if some wave of head x keeps the block it last voted
        // on (a vote: bit 0 first key half skipped; bits 1/2 second half
        // skipped after a skipped / kept first half). One 16-byte LDS read,
        // issued next to the wave's own vote reads.
        auto head_keeps = [&](int x) -> int {
            const u32x4 v = *(const u32x4 *)&sVote[x * WPH];
            auto group_skips = [&](uint32_t vall) {
                const bool ska = (vall & 1) != 0;
                const bool skb = KH ? (((ska ? vall >> 1 : vall >> 2) & 1) != 0) : ska;
                return ska && skb;
            };
            const bool sk = (KH && p.half_vote != 0) ? group_skips(v[0] & v[1]) && group_skips(v[2] & v[3])
                                                     : group_skips(v[0] & v[1] & v[2] & v[3]);
            return __builtin_amdgcn_readfirstlane(sk ? 0 : 1);
        };
        auto v_sparse = [&](int j, auto after_vote) {
            // the votes of this wave's head, or of its half-tile's two waves
            // A wave whose own vote keeps the whole block (both halves under key-half
            // decisions: the second against the first half kept) knows the decision,
            // since the head ANDs its waves' skip votes: it reads no vote words.
            int vall = 0, hk = 1;
            if ((my_vote & (KH ? 5 : 1)) != 0) {
                const int vmask = (KH && p.half_vote != 0) ? 3 << (wq & 2) : (1 << WPH) - 1;
                vall = 7;
#pragma unroll
                for (int y = 0; y < WPH; ++y)
                    if ((vmask >> y) & 1) vall &= sVote[hl * WPH + y];
                hk = head_keeps(hl);
                vall = __builtin_amdgcn_readfirstlane(vall);
            }
            bool ska, skb;  // decisions on the two key halves
            if constexpr (KH) {
                ska = (vall & 1) != 0;
                skb = ((ska ? vall >> 1 : vall >> 2) & 1) != 0;
                if (2 * j < nlog) log_decision(p, lg, bm_row, 2 * j, nlog, ska, lane == 0);
                if (2 * j + 1 < nlog) log_decision(p, lg, bm_row, 2 * j + 1, nlog, skb, lane == 0);
            } else {
                ska = skb = (vall & 1) != 0;
                if (j < nlog) log_decision(p, lg, bm_row, j, nlog, ska, lane == 0);
            }
            const bool sk = ska && skb;
            pend = !sk;
            after_vote(hk);
            if (!sk || (p.flags & BSP_FLAG_EXP_SKIPPED) != 0) {
                float alpha, rs0 = 0.f, rs1 = 0.f;
                bool resc;
                const float mc = new_reference(fmaxf(ska ? -INFINITY : mloc_a, skb ? -INFINITY : mloc_b), j * BK, alpha,
                                               resc);
                // a skipped half's exponentials are taken against +inf: zero probabilities, zero sum
                const float mca = ska ? INFINITY : mc, mcb = skb ? INFINITY : mc;
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    const float mce = (e >> 4) < MT / 2 ? mca : mcb;
                    sacc[e >> 4][e & 15] = __builtin_amdgcn_exp2f(fmaf(sacc[e >> 4][e & 15], c, -mce));
                    if (e & 1) {
                        rs0 += sacc[(e - 1) >> 4][(e - 1) & 15];
                        rs1 += sacc[e >> 4][e & 15];
                    }
                }
                float rs = rs0 + rs1;
                rs = halves_sum(rs);
                if (resc) {
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
                }
                l_run += rs;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int i = 0; i < 8; ++i) pprev[2 * mt + u][i] = (__bf16)sacc[mt][8 * u + i];
            } else {
#pragma unroll
                for (int cc = 0; cc < PC; ++cc) pprev[cc] = bf16x8{};
            }
        };

        using T_ = std::true_type;
        using F_ = std::false_type;
        const int n = nblk;
        if constexpr (SPP) {
            // V-load skip. V_j is needed by head 0 in interval 2j + 2 and by
            // head 1 in interval 2j + 3; it is copied once some head keeps
            // block j, by the waves of that head alone (each wave its own share
            // of the block and that of the other head's wave of the same index),
            // right after they decide in their vector phase: head 0 in interval
            // 2j + 1, when it keeps j; else head 1 in interval 2j + 2 (a late
            // copy), when it keeps j. The copying waves wait for their copies
            // before the barrier that ends the interval. When both heads skip j,
            // V_j is never loaded. Head 0 publishes its decision in sHead during
            // interval 2j + 1, and head 1 reads it in interval 2j + 2, so no
            // wave reads another head's votes in its matrix phase. Block 0 is
            // never skipped: V_0 goes with K_1 in interval 0.
            using N0 = std::integral_constant<int, 0>;
            using NK = std::integral_constant<int, CI>;        // this wave's share of K_{j+1}
            using NKV = std::integral_constant<int, 2 * CI>;   // ... and of V_j
            const bool v_all = (p.flags & BSP_FLAG_LOAD_SKIPPED_V) != 0;  // ablation: copy every V
            const int dwo = hl == 0 ? WPH : -WPH;  // the other head's wave of the same index
            auto copy_v_head = [&](int j) {
#pragma unroll
                for (int i = 0; i < CI; ++i) {
                    issue_copy(j, CI + i);
                    if constexpr (F8) copy_one(vg, vstb, j * BK, sV8[j & (NV8 - 1)], false, i, dwo);
                    else copy_one(vg, vstb, j * BK, sV[j & 1], true, i, dwo);
                }
            };
            auto land_v_head = [&](int j) {  // fp8: widen both shares
                if constexpr (F8) {
                    widen_v(sV[j & 1], j & (NV8 - 1));
                    widen_v(sV[j & 1], j & (NV8 - 1), dwo);
                }
            };
            if (hl == 0) {
                qk_vote(0, NKV{});                        // interval 0: K_1, V_0
                __syncthreads();
                v_sparse(0, [&](int) {                    // interval 1 (block 0 is kept)
                    if (wq == 0 && lane == 0) sHead = 1;
                });
                wait_vmem_all();
                land_v(0);
                __syncthreads();
                int h0k = 1;
                for (int j = 1; j < n; ++j) {
                    if (pend) pv_part(j);                 // interval 2j: PV_{j-1}, QK_j with K_{j+1}
                    qk_vote(j, NK{});
                    __syncthreads();
                    bool cp = false;                      // interval 2j + 1: vector phase of block j
                    v_sparse(j, [&](int hk) {
                        h0k = hk;
                        if (wq == 0 && lane == 0) sHead = hk;
                        cp = hk != 0 || v_all;
                        if (cp) copy_v_head(j);
                    });
                    wait_vmem_all();
                    if (cp) land_v_head(j);
                    __syncthreads();
                }
                if (pend) pv_part(n);                     // interval 2n: PV_{n-1}
                // head 1 copies V_{n-1} late when it keeps the block head 0 skipped (same test on both heads)
                if (h0k == 0 && !v_all && head_keeps(1) != 0) __syncthreads();
            } else {
#pragma unroll
                for (int i = 0; i < 2 * CI; ++i) issue_copy(0, i);  // interval 0: K_1, V_0
                __syncthreads();
                qk_vote(0, N0{});                         // interval 1
                wait_vmem_all();
                land_v(0);
                __syncthreads();
                for (int j = 1; j < n; ++j) {
                    // interval 2j: vector phase of block j - 1; K_{j+1}, and V_{j-1} when this head keeps
                    // the block head 0 skipped
                    bool late = false;
                    const int h0k_lds = sHead;            // read early: its wait falls after the decision
                    v_sparse(j - 1, [&](int hk) {
                        const int h0k = __builtin_amdgcn_readfirstlane(h0k_lds);
#pragma unroll
                        for (int i = 0; i < CI; ++i) issue_copy(j, i);
                        late = hk != 0 && h0k == 0 && !v_all;
                        if (late) copy_v_head(j - 1);
                    });
                    if (late) {
                        wait_vmem_all();
                        land_v_head(j - 1);
                    }
                    __syncthreads();
                    if (pend) pv_part(j);                 // interval 2j + 1: PV_{j-1}, QK_j
                    qk_vote(j, N0{});
                    wait_vmem_all();
                    __syncthreads();
                }
                bool late = false;                        // interval 2n: vector phase of block n-1
                const int h0k_lds = sHead;
                v_sparse(n - 1, [&](int hk) {
                    late = hk != 0 && __builtin_amdgcn_readfirstlane(h0k_lds) == 0 && !v_all;
                    if (late) copy_v_head(n - 1);
                });
                if (late) {
                    wait_vmem_all();
                    land_v_head(n - 1);
                    __syncthreads();
                }
                if (pend) pv_part(n);                     // interval 2n + 1
            }
        } else if (hl == 0) {
            m_phase(0, F_{}, T_{}, T_{});                 // interval 0
            __syncthreads();
            v_phase(0, F_{}, 0);                          // interval 1
            wait_vmem_all();
            land_v(0);
            __syncthreads();
            for (int j = 1; j < n; ++j) {
                m_phase(j, T_{}, T_{}, T_{});             // interval 2j
                __syncthreads();
                v_phase(j, F_{}, 0);                      // interval 2j + 1
                wait_vmem_all();
                land_v(j);
                __syncthreads();
            }
            m_phase(n, T_{}, F_{}, F_{});                 // interval 2n: PV_{n-1}
        } else {
#pragma unroll
            for (int i = 0; i < 2 * CI; ++i) issue_copy(0, i);  // interval 0: K_1, V_0
            __syncthreads();
            m_phase(0, F_{}, T_{}, F_{});                 // interval 1
            wait_vmem_all();
            land_v(0);
            __syncthreads();
            for (int j = 1; j < n; ++j) {
                v_phase(j - 1, T_{}, j);                  // interval 2j (copies of K_{j+1}, V_j)
                __syncthreads();
                m_phase(j, T_{}, T_{}, F_{});             // interval 2j + 1
                wait_vmem_all();
                land_v(j);
                __syncthreads();
            }
            v_phase(n - 1, F_{}, 0);                      // interval 2n
            m_phase(n, T_{}, F_{}, F_{});                 // interval 2n + 1: PV_{n-1}
        }
        pend = false;
        v_prev = false;
    } else if constexpr (DENSE) {
        // ---- dense mode: every block is kept. Block 0 has no pending PV; every
        // later block runs the PV product of the previous block interleaved with
        // its own exponentials and row sum: group g is PV MFMA g (V operand read
        // two MFMAs ahead) followed by the exponentials of elements EPG*g ..
        // EPG*g + EPG - 1 and the row sum of the previous group's elements, so the
        // matrix cores and the vector ALU work side by side. The fences keep this
        // order; the loop body has no branches, so the compiler keeps one register
        // assignment for the accumulators.
        {
            const float mloc = qk_phase(0);
            __syncthreads();  // B1: every wave is done with QK_0
            if constexpr (F8) copy_block(vg, vstb, 0, sV8[0], false);
            else copy_block(vg, vstb, 0, sV[0], true);
            float alpha;
            bool resc;
            const float mc = new_reference(mloc, 0, alpha, resc);
            finish_block(exp_sum(mc), alpha, resc);
            wait_vmem_leave<CI>();
            __syncthreads();  // B2: K_1 in LDS
        }
        for (int j = 1; j < nblk; ++j) {
            const int cur = j & 1;
            const float mloc = qk_phase(j);
            // V_{j-1} must be in LDS before B1; K_{j+1} may still fly.
            wait_vmem_leave<CI>();
            widen_v(sV[0]);
            __syncthreads();  // B1
            if constexpr (F8) copy_block(vg, vstb, j * BK, sV8[0], false);
            else copy_block(vg, vstb, j * BK, sV[cur], true);
            float alpha;
            bool resc;
            const float mc = new_reference(mloc, j * BK, alpha, resc);
            finish_block(fused_pv_exp(sV[F8 ? 0 : (cur ^ 1)], mc), alpha, resc);
            // B2: K_{j+1} is in LDS (loads complete in issue order; V_j, issued last, may still fly).
            wait_vmem_leave<CI>();
            __syncthreads();
        }
        pend = true;
        v_prev = true;
    } else {
        // ---- sparse mode: per block, the tile-wide vote decides skip or keep.
        for (int j = 0; j < nblk; ++j) {
            const int kb = j * BK;
            const int cur = j & 1;
            const float mloc = qk_phase(j);
            // skip decision: every valid row of the head's tile must have gap > lambda
            {
                const bool ok = !valid || (mloc == -INFINITY) || (m_dec - mloc > lam_raw);
                const int wall = __all(ok);
                if (lane == 0) sVote[w] = wall;
            }
            // V_{j-1} (copied during the previous block) must be in LDS before B1; K_{j+1} may still fly.
            if (v_prev) {
                wait_vmem_leave<CI>();
                widen_v(sV[0]);
            }
            __syncthreads();  // B1: votes and V_{j-1} visible; every wave is done with QK_j
            bool skip = false;
            bool any_keep = false;
#pragma unroll
            for (int x = 0; x < HPW; ++x) {
                bool sk = true;
#pragma unroll
                for (int y = 0; y < WPH; ++y) sk = sk && (sVote[x * WPH + y] != 0);
                if (x == hl) skip = sk;
                any_keep = any_keep || !sk;
            }
            if (wq == 0) log_decision(p, lg, bm_row, j, nblk, skip, lane == 0);
            // ablation: copy V also for blocks every head skips
            any_keep = any_keep || (p.flags & BSP_FLAG_LOAD_SKIPPED_V) != 0;
            if (any_keep) {
                if constexpr (F8) copy_block(vg, vstb, kb, sV8[0], false);
                else copy_block(vg, vstb, kb, sV[cur], true);
            }
            // Exponentials in place, then the pending PV, then row sum, rescale and
            // the bf16 probabilities (the fused order of the dense loop does not fit
            // the registers next to the skip branches). Ablation: a skipped block's
            // exponentials are computed against the unchanged reference and dropped.
            float alpha = 1.f;
            bool resc = false;
            if (!skip || (p.flags & BSP_FLAG_EXP_SKIPPED) != 0) {
                const float mc = skip ? m_ref * c : new_reference(mloc, kb, alpha, resc);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[mt][i] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][i], c, -mc));
            }
            if (pend) pv_block(pprev, sV[F8 ? 0 : (cur ^ 1)]);
            if (!skip) {
                float rs = 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) rs += sacc[mt][i];
                rs = halves_sum(rs);
                if (resc) {
                    l_run *= alpha;
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
                }
                l_run += rs;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int i = 0; i < 8; ++i) pprev[2 * mt + u][i] = (__bf16)sacc[mt][8 * u + i];
            }
            pend = !skip;
            v_prev = any_keep;

            // B2: K_{j+1} is in LDS (loads complete in issue order; V_j, issued last, may still fly).
            if (any_keep) wait_vmem_leave<CI>();
            else wait_vmem_all();
            __syncthreads();
        }
    }
    wait_vmem_all();  // also the copy past the last K block, before the workgroup ends
    if (v_prev) {
        widen_v(sV[0]);
        __syncthreads();
    }
    if (pend) pv_block(pprev, sV[F8 ? 0 : ((nblk - 1) & 1)]);

    // ---- epilogue: normalise, store O (bf16) and LSE (natural log). The output
    // fields are read here from the kernel argument segment (BSP_LATE_ARG), so
    // they are loaded at this point instead of occupying scalar registers
    // across the loop.
    if (valid) {
        const float inv = osc / l_run;
        __bf16 *op = (__bf16 *)BSP_LATE_ARG(FwdParams, o) + (int64_t)(base + qrow) * BSP_LATE_ARG(FwdParams, o_st) +
                     (int64_t)h * BSP_LATE_ARG(FwdParams, o_sh);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const bf16x4 x = {(__bf16)(oacc[dt][4 * g4 + 0] * inv), (__bf16)(oacc[dt][4 * g4 + 1] * inv),
                                  (__bf16)(oacc[dt][4 * g4 + 2] * inv), (__bf16)(oacc[dt][4 * g4 + 3] * inv)};
                *(bf16x4 *)(op + 32 * dt + 8 * g4 + 4 * hh) = x;
            }
        float *lse = BSP_LATE_ARG(FwdParams, lse);
        if (hh == 0 && lse != nullptr)
            lse[(int64_t)h * BSP_LATE_ARG(FwdParams, lse_sh) + base + qrow] = (m_ref * c + __log2f(l_run)) * kLn2;
    }
    // wave 0 of the head adds the tile's visited blocks; the waves that recorded
    // decisions add their skips (wave 2 as well under half-tile votes)
    if (KH && lane == 0 && wq == 2 && BSP_LATE_ARG(FwdParams, half_vote) != 0 && lg.nskip != 0) {
        unsigned long long *c0 = BSP_LATE_ARG(FwdParams, skip_count), *c2 = BSP_LATE_ARG(FwdParams, seq_skip);
        if (c0) atomicAdd(&c0[h], (unsigned long long)lg.nskip);
        if (c2) atomicAdd(&c2[s], (unsigned long long)lg.nskip);
    }
    if (wq == 0 && lane == 0) {
        unsigned long long *c0 = BSP_LATE_ARG(FwdParams, skip_count), *c1 = BSP_LATE_ARG(FwdParams, visited_count);
        unsigned long long *c2 = BSP_LATE_ARG(FwdParams, seq_skip), *c3 = BSP_LATE_ARG(FwdParams, seq_visited);
        if (c0) atomicAdd(&c0[h], (unsigned long long)lg.nskip);
        int vis = nblk;
        if (p.acct_bq > 0) {  // the caller's query tiles inside this one, each with its causal key blocks
            vis = 0;
            for (int r0 = t * BQ; r0 < r1; r0 += p.acct_bq) vis += (off + min(r0 + p.acct_bq, L) - 1) / p.acct_bk + 1;
        }
        if (c1) atomicAdd(&c1[h], (unsigned long long)vis);
        if (c2) atomicAdd(&c2[s], (unsigned long long)lg.nskip);
        if (c3) atomicAdd(&c3[s], (unsigned long long)vis);
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: QK^T and PV on v_mfma_f32_32x32x2_f32 (one element per lane
// per operand, so V needs no transpose).
// ---------------------------------------------------------------------------
template <int D, int BQ, int BK, bool PAGED>
__global__ void __launch_bounds__(BQ * 2) fwd_f32(FwdParams p) {
    constexpr int NW = BQ / 32;
    constexpr int NT = NW * 64;
    constexpr int KS = D / 2;
    constexpr int MT = BK / 32;
    constexpr int DT = D / 32;
    constexpr int STR = D + 1;
    __shared__ float sK[BK * STR];
    __shared__ float sV[BK * STR];
    __shared__ __attribute__((aligned(16))) int sVote[NW];
    __shared__ int sHead;  // two-head sparse schedule: 1 if head 0 keeps the block it decided last

    int s, t, h;
    decode_item(p, s, t, h);
    const int base = p.cu[s];
    const int L = p.cu[s + 1] - base;  // query rows of the sequence (its chunk)
    if (t * BQ >= L) return;
    const int kbase = p.cu_k ? p.cu_k[s] : base;
    const int Lk = p.cu_k ? p.cu_k[s + 1] - kbase : L;  // keys
    const int off = Lk - L;            // query row r sits at key position off + r
    if (off < 0) return;               // caller error: nothing written

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int ln = lane & 31;
    const int hh = lane >> 5;
    const int g = h / p.G;
    const int r1 = min((t + 1) * BQ, L);
    const int nblk = (off + r1 - 1) / BK + 1;
    const int q0 = t * BQ + w * 32;
    const int qrow = q0 + ln;
    const bool valid = qrow < L;
    const int qpos = off + qrow;
    const int64_t bm_row = ((int64_t)h * p.n_seqs + s) * p.T_bm + t;
    const float lam_raw = p.lam_seq == nullptr ? p.lam_raw
                          : (p.lam_seq[s] == INFINITY ? INFINITY : p.lam_seq[s] / p.scale);

    const float *qg = (const float *)p.q;
    const float *kg = (const float *)p.k;
    const float *vg = (const float *)p.v;

    float qf[KS];  // lane holds Q[qrow][2ks + hh]
    {
        const float *qp = qg + (int64_t)(base + (valid ? qrow : 0)) * p.q_st + (int64_t)h * p.q_sh + hh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = valid ? qp[2 * ks] : 0.f;
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
    SkipLog lg;

    for (int j = 0; j < nblk; ++j) {
        const int kb = j * BK;
        __syncthreads();
        for (int c = tid; c < BK * D / 4; c += NT) {
            const int r = c / (D / 4);
            const int c4 = c % (D / 4);
            const int kk = kb + r;
            f32x4 x{};
            if (kk < Lk) x = *(const f32x4 *)(kg + kv_row<PAGED>(p, s, kbase, kk, p.k_st) + (int64_t)g * p.k_sh + 4 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) sK[r * STR + 4 * c4 + e] = x[e];
        }
        __syncthreads();

        f32x16 sacc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x16 acc{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[(32 * mt + ln) * STR + 2 * ks + hh], qf[ks], acc, 0, 0, 0);
            sacc[mt] = acc;
        }
        if (kb + BK - 1 > off + q0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kb + 32 * mt + 8 * (i >> 2) + 4 * hh + (i & 3);
                    if (key > qpos) sacc[mt][i] = -INFINITY;
                }
        }
        float mloc = wave_max16(sacc[0]);
#pragma unroll
        for (int mt = 1; mt < MT; ++mt) mloc = fmaxf(mloc, wave_max16(sacc[mt]));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));

        const bool ok = !valid || (mloc == -INFINITY) || (m_run - mloc > lam_raw);
        const int wall = __all(ok);
        if (lane == 0) sVote[w] = wall;
        __syncthreads();
        bool skip = true;
#pragma unroll
        for (int x = 0; x < NW; ++x) skip = skip && (sVote[x] != 0);
        log_decision(p, lg, bm_row, j, nblk, skip, tid == 0);
        if (!skip || (p.flags & BSP_FLAG_LOAD_SKIPPED_V) != 0) {
            for (int c = tid; c < BK * D / 4; c += NT) {
                const int r = c / (D / 4);
                const int c4 = c % (D / 4);
                const int kk = kb + r;
                f32x4 x{};
                if (kk < Lk) x = *(const f32x4 *)(vg + kv_row<PAGED>(p, s, kbase, kk, p.v_st) + (int64_t)g * p.v_sh + 4 * c4);
#pragma unroll
                for (int e = 0; e < 4; ++e) sV[r * STR + 4 * c4 + e] = x[e];
            }
        }
        if (skip) {
            if ((p.flags & BSP_FLAG_EXP_SKIPPED) != 0) {  // ablation: exponentials computed and dropped
                const float mc = m_run * p.c_log2;
                float sink = 0.f;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sink += __builtin_amdgcn_exp2f(fmaf(sacc[mt][i], p.c_log2, -mc));
                asm volatile("" ::"v"(sink));
            }
            continue;
        }

        const float m_new = fmaxf(m_run, mloc);
        const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * p.c_log2);
        const float mc = m_new * p.c_log2;
        float rs = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = __builtin_amdgcn_exp2f(fmaf(sacc[mt][i], p.c_log2, -mc));
                sacc[mt][i] = e;
                rs += e;
            }
        rs += __shfl_xor(rs, 32);
        l_run = alpha * l_run + rs;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        __syncthreads();

        // O^T += V^T P^T: contraction step (mt, i) pairs key 32mt + 8(i/4) + 4hh + i%4 of both halves
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 32 * mt + 8 * (i >> 2) + 4 * hh + (i & 3);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[key * STR + 32 * dt + ln], sacc[mt][i], oacc[dt],
                                                                    0, 0, 0);
                }
    }

    if (valid) {
        const float inv = 1.f / l_run;
        float *op = (float *)p.o + (int64_t)(base + qrow) * p.o_st + (int64_t)h * p.o_sh;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = {oacc[dt][4 * g4 + 0] * inv, oacc[dt][4 * g4 + 1] * inv, oacc[dt][4 * g4 + 2] * inv,
                                 oacc[dt][4 * g4 + 3] * inv};
                *(f32x4 *)(op + 32 * dt + 8 * g4 + 4 * hh) = x;
            }
        if (hh == 0 && p.lse != nullptr)
            p.lse[(int64_t)h * p.lse_sh + base + qrow] = (m_run * p.c_log2 + __log2f(l_run)) * kLn2;
    }
    if (tid == 0) {
        if (p.skip_count) atomicAdd(&p.skip_count[h], (unsigned long long)lg.nskip);
        if (p.visited_count) atomicAdd(&p.visited_count[h], (unsigned long long)nblk);
        if (p.seq_skip) atomicAdd(&p.seq_skip[s], (unsigned long long)lg.nskip);
        if (p.seq_visited) atomicAdd(&p.seq_visited[s], (unsigned long long)nblk);
    }
}

// ---------------------------------------------------------------------------
// Decoding step: one new query row per sequence against all of its keys
// (the guide's decode-phase use of the same rule). The row's causal window is
// every key, so the tile-wide rule reduces to one row: block j is skipped
// when max(M_0 .. M_{j-1}) - M_j > lambda, with M_j the block's largest score.
// That prefix maximum does not depend on earlier decisions (a skipped block
// never holds a larger score), so the key range of a sequence splits into
// chunks that decide independently and exactly:
//   dec_scores:  S = q.k for every key (dequantised), block maxima M;
//   dec_pv:      per chunk, the prefix max before the chunk and the
//                sequence's overall max Mall (from M), the decisions, and
//                sum p*v, sum p over kept blocks with p = exp(scale*(S - Mall));
//   dec_combine: o = sum over chunks / sum of p, lse = scale*Mall + ln(sum p).
// The kernels are bound by HBM bytes: K once, V for blocks some query head of
// the KV group keeps, the scores written and read once. All vector ALU: four
// query heads per KV head are too few rows for the matrix cores.
// ---------------------------------------------------------------------------
constexpr int kDecRows = 8;    // V row loads per wave in flight in the decode PV kernel
constexpr int kDecRowsS = 4;   // K row loads per batch in the decode score kernel (two batches in flight)
constexpr int kDecMaxC = 256;  // key blocks per decode chunk, at most

struct DecParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh;  // elements; q and o rows are sequences
    int64_t lse_sh;                // elements between heads of lse (= n_seqs)
    int64_t total_k;               // score rows per head (= cu_k[n_seqs])
    const int32_t *cu_k;           // key offsets per sequence (packed rows; score rows)
    const int32_t *table;          // paged: block table, else NULL
    int32_t max_pages, page_shift;
    uint32_t *bitmap;
    unsigned long long *skip_count, *visited_count, *seq_skip, *seq_visited;
    int32_t n_seqs, W, J_max, n_chunks, C, BK, Hq, Hkv, G;
    float c_log2, lam_raw, scale;  // lam_raw: lambda / scale (scores are unscaled dot products)
    const float *lam_seq;
    const float *q_scale, *k_scale, *v_scale;
    uint32_t flags;
    float *S;     // [Hkv][total_k][GP]: scores of the GP (padded) query heads of a KV head, key-major
    float *M;     // [Hq][n_seqs][J_max]
    float *part;  // [Hq][n_seqs][n_chunks][D + 1]: sum p*v over the chunk, then sum p
};

// Sum over the LPR consecutive lanes that hold one K/V row (LPR = 8 or 16),
// through DPP: quad exchanges (lane ^ 1, lane ^ 2), then the mirror within
// each 8 lanes and, for 16, within each 16 lanes. Every lane gets the sum.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    auto dpp = [](float v, int ctrl) -> float {
        switch (ctrl) {
            case 0: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
            case 1: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
            case 2: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
            default: return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
        }
    };
    x += dpp(x, 0);
    x += dpp(x, 1);
    x += dpp(x, 2);
    if constexpr (LPR == 16) x += dpp(x, 3);
    return x;
}

// Row sums of NH values at once (one DPP step for every value before the next
// step, so no step waits on the one just issued).
template <int LPR, int NH>
__device__ __forceinline__ void row_sums(float *x) {
    auto step = [&](int ctrl) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const float xh = x[h];
            const int v = __builtin_bit_cast(int, xh);
            int y;
            if (ctrl == 0) y = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true);        // lane ^ 1
            else if (ctrl == 1) y = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true);   // lane ^ 2
            else if (ctrl == 2) y = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);  // mirror in 8
            else y = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true);                 // mirror in 16
            x[h] += __builtin_bit_cast(float, y);
        }
    };
    step(0);
    step(1);
    step(2);
    if constexpr (LPR == 16) step(3);
}

// 16 bytes of a row as packed bf16 pairs: 4 words for bf16, 8 for e4m3 codes
// (each pair widened exactly).
template <bool F8>
__device__ __forceinline__ void pairs16(const u32x4 x, bf16x2 *w) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (F8) {
            w[2 * i] = __builtin_bit_cast(bf16x2, fp8x2_to_bf16x2<false>(x[i]));
            w[2 * i + 1] = __builtin_bit_cast(bf16x2, fp8x2_to_bf16x2<true>(x[i]));
        } else {
            // (through a scalar: a bit_cast applied directly to a vector element
            // reads element 0 for every i with this compiler)
            const uint32_t xi = x[i];
            w[i] = __builtin_bit_cast(bf16x2, xi);
        }
    }
}

// 16 bytes of a row as fp32: 8 bf16 values, or 16 e4m3 codes (widened exactly).
template <bool F8>
__device__ __forceinline__ void widen16(const u32x4 x, float *f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (F8) {
            const uint32_t lo = fp8x2_to_bf16x2<false>(x[i]), hi = fp8x2_to_bf16x2<true>(x[i]);
            f[4 * i + 0] = __builtin_bit_cast(float, lo << 16);
            f[4 * i + 1] = __builtin_bit_cast(float, lo & 0xffff0000u);
            f[4 * i + 2] = __builtin_bit_cast(float, hi << 16);
            f[4 * i + 3] = __builtin_bit_cast(float, hi & 0xffff0000u);
        } else {
            f[2 * i + 0] = __builtin_bit_cast(float, x[i] << 16);
            f[2 * i + 1] = __builtin_bit_cast(float, x[i] & 0xffff0000u);
        }
    }
}

// Byte address of key `key` of sequence s in K or V of KV head g (base already at head g).
template <bool PAGED>
__device__ __forceinline__ const char *dec_row(const DecParams &p, const char *base_g, int64_t stb, int s, int kbase,
                                               int key) {
    if constexpr (PAGED) {
        const int pg = p.table[(int64_t)s * p.max_pages + min(key >> p.page_shift, p.max_pages - 1)];
        return base_g + (((int64_t)pg << p.page_shift) + (key & ((1 << p.page_shift) - 1))) * stb;
    } else {
        return base_g + (int64_t)(kbase + key) * stb;
    }
}

// Work item of the decode kernels: (sequence, chunk of C key blocks, KV head),
// KV head fastest: neighbouring workgroups read the same key rows (which hold
// all KV heads side by side), so DRAM pages are read once, not once per head.
__device__ __forceinline__ bool dec_item(const DecParams &p, int &s, int &g, int &c, int &kbase, int &Lk, int &nblk,
                                         int &j0, int &j1) {
    int item = blockIdx.x;
    g = item % p.Hkv;
    item /= p.Hkv;
    c = item % p.n_chunks;
    s = item / p.n_chunks;
    kbase = p.cu_k[s];
    Lk = p.cu_k[s + 1] - kbase;
    nblk = Lk > 0 ? min((Lk + p.BK - 1) / p.BK, p.J_max) : 0;
    j0 = c * p.C;
    j1 = min(j0 + p.C, nblk);
    return j0 < j1;
}

// Scores and block maxima. 4 waves; a row of K is read by LPR lanes, 16 bytes
// each, and a wave covers RPW rows per load.
template <int IN, int D, bool PAGED, int GP>
__global__ void __launch_bounds__(256) dec_scores(DecParams p) {
    constexpr bool F8 = IN == BSP_FP8_E4M3;
    constexpr int ES = F8 ? 1 : 2;
    constexpr int LPR = D * ES / 16;
    constexpr int EPL = 16 / ES;
    constexpr int RPW = 64 / LPR;
    static_assert(LPR == 8 || LPR == 16, "a row is 8 or 16 lanes");
    int s, g, c, kbase, Lk, nblk, j0, j1;
    const bool work = dec_item(p, s, g, c, kbase, Lk, nblk, j0, j1);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = p.G;
    if (c == 0) {
        // outputs of this (sequence, KV head), before any early exit: its bitmap rows, the
        // query heads' counts (by sequence 0) and the sequence's counts (by KV head 0).
        // dec_pv, the next kernel, then adds to them.
        if (p.bitmap != nullptr)
            for (int i = tid; i < G * p.W; i += 256)
                p.bitmap[((int64_t)(g * G + i / p.W) * p.n_seqs + s) * p.W + i % p.W] = 0u;
        if (s == 0 && tid < G) {
            if (p.skip_count) p.skip_count[g * G + tid] = 0ull;
            if (p.visited_count) p.visited_count[g * G + tid] = 0ull;
        }
        if (g == 0 && tid == 0) {
            if (p.seq_skip) p.seq_skip[s] = 0ull;
            if (p.seq_visited) p.seq_visited[s] = 0ull;
        }
    }
    if (!work) return;
    const int sub = lane % LPR, rw = lane / LPR;
    constexpr int NPR = EPL / 2;  // bf16 pairs per lane per row
    bf16x2 qp[GP][NPR];
    float sqk[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        const int hq = g * G + (h < G ? h : 0);
        const u32x4 x = *(const u32x4 *)((const char *)p.q + ((int64_t)s * p.q_st + (int64_t)hq * p.q_sh) * ES + 16 * sub);
        pairs16<F8>(x, qp[h]);
        sqk[h] = F8 ? p.q_scale[hq] * p.k_scale[g] : 1.f;
    }
    const char *kg = (const char *)p.k + (int64_t)g * p.k_sh * ES;
    const int64_t kst = p.k_st * ES;
    float *Sg = p.S + ((int64_t)g * p.total_k + kbase) * GP;
    // The chunk's blocks go round-robin to the 4 waves; a wave reduces its block
    // alone. A wave's blocks are taken as one sequence of batches of kDecRowsS row
    // loads (rows past a block re-read its last row), software-pipelined: the
    // loads of the next batch are issued before the current one is computed.
    constexpr int R = kDecRowsS;
    constexpr int RB = RPW * R;  // rows per batch
    auto block_rows = [&](int j) { return min(p.BK, Lk - j * p.BK); };
    auto issue = [&](u32x4 (&xs)[R], int j, int r0) {
        const int kb = j * p.BK, rows = block_rows(j);
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int r = r0 + RPW * u + rw;
            xs[u] = *(const u32x4 *)(dec_row<PAGED>(p, kg, kst, s, kbase, kb + min(r, rows - 1)) + 16 * sub);
        }
    };
    float bmax[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) bmax[h] = -INFINITY;
    // scores of one batch; after the last batch of a block, the block maximum
    auto consume = [&](const u32x4 (&xs)[R], int j, int r0) {
        const int kb = j * p.BK, rows = block_rows(j);
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int r = r0 + RPW * u + rw;
            const bool ok = r < rows;
            bf16x2 kp[NPR];
            pairs16<F8>(xs[u], kp);
            float d[GP];
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                d[h] = 0.f;
#pragma unroll
                for (int i = 0; i < NPR; ++i) d[h] = __builtin_amdgcn_fdot2_f32_bf16(kp[i], qp[h][i], d[h], false);
            }
            row_sums<LPR, GP>(d);
            float mine = 0.f;  // lane sub < GP stores head sub's score of the row
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                d[h] *= sqk[h];
                bmax[h] = fmaxf(bmax[h], ok ? d[h] : -INFINITY);
                mine = sub == h ? d[h] : mine;
            }
            if (ok && sub < GP) Sg[(int64_t)(kb + r) * GP + sub] = mine;
        }
        if (r0 + RB >= rows) {
#pragma unroll
            for (int h = 0; h < GP; ++h) {
#pragma unroll
                for (int m = LPR; m < 64; m <<= 1) bmax[h] = fmaxf(bmax[h], __shfl_xor(bmax[h], m));
            }
            if (lane < G) {
                float m = bmax[0];
#pragma unroll
                for (int h = 1; h < GP; ++h) m = lane == h ? bmax[h] : m;
                p.M[((int64_t)(g * G + lane) * p.n_seqs + s) * p.J_max + j] = m;
            }
#pragma unroll
            for (int h = 0; h < GP; ++h) bmax[h] = -INFINITY;
        }
    };
    auto advance = [&](int &j, int &r0) {
        r0 += RB;
        if (r0 >= block_rows(j)) {
            j += 4;
            r0 = 0;
        }
    };
    int j = j0 + w, r0 = 0;
    u32x4 xa[R], xb[R];
    if (j < j1) issue(xa, j, 0);
    while (j < j1) {  // two batches per trip, so that the buffers keep their registers
        const int ja = j, ra = r0;
        advance(j, r0);
        if (j < j1) issue(xb, j, r0);
        consume(xa, ja, ra);
        if (j >= j1) break;
        const int jb = j, rb = r0;
        advance(j, r0);
        if (j < j1) issue(xa, j, r0);
        consume(xb, jb, rb);
    }
}

// o and lse of one (sequence, query head) from the chunk partials: four waves
// (the whole workgroup) take every fourth chunk, lanes take dimensions, then
// wave 0 adds up and stores.
template <int D>
__device__ __forceinline__ void dec_combine_head(const DecParams &p, int s, int hq, int nblk) {
    constexpr int DL = D / 64;  // dimensions per lane
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    __shared__ float sm[4];
    __shared__ float sa[4][D + 1];
    const float *Mh = p.M + ((int64_t)hq * p.n_seqs + s) * p.J_max;
    float mall = -INFINITY;
    for (int j = tid; j < nblk; j += 256) mall = fmaxf(mall, Mh[j]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) mall = fmaxf(mall, __shfl_xor(mall, m));
    if (lane == 0) sm[w] = mall;
    const int nch = (nblk + p.C - 1) / p.C;
    const float *ph = p.part + ((int64_t)hq * p.n_seqs + s) * p.n_chunks * (D + 1);
    float l = 0.f;
    float a[DL] = {};
    int c = w;
    for (; c + 12 < nch; c += 16) {  // four chunks of this wave in flight
        float lv[4], av[4][DL];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float *pc = ph + (int64_t)(c + 4 * u) * (D + 1);
            lv[u] = pc[D];
#pragma unroll
            for (int i = 0; i < DL; ++i) av[u][i] = pc[lane + 64 * i];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            l += lv[u];
#pragma unroll
            for (int i = 0; i < DL; ++i) a[i] += av[u][i];
        }
    }
    for (; c < nch; c += 4) {
        const float *pc = ph + (int64_t)c * (D + 1);
        l += pc[D];
#pragma unroll
        for (int i = 0; i < DL; ++i) a[i] += pc[lane + 64 * i];
    }
#pragma unroll
    for (int i = 0; i < DL; ++i) sa[w][lane + 64 * i] = a[i];
    if (lane == 0) sa[w][D] = l;
    __syncthreads();
    if (w == 0) {
        mall = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
        l = (sa[0][D] + sa[1][D]) + (sa[2][D] + sa[3][D]);
        const float osc = p.v_scale != nullptr ? p.v_scale[hq / p.G] : 1.f;
        const float inv = osc / l;
        __bf16 *op = (__bf16 *)p.o + (int64_t)s * p.o_st + (int64_t)hq * p.o_sh;
#pragma unroll
        for (int i = 0; i < DL; ++i) {
            const int d = lane + 64 * i;
            op[d] = (__bf16)(((sa[0][d] + sa[1][d]) + (sa[2][d] + sa[3][d])) * inv);
        }
        if (lane == 0 && p.lse != nullptr) p.lse[(int64_t)hq * p.lse_sh + s] = (mall * p.c_log2 + __log2f(l)) * kLn2;
    }
    __syncthreads();  // sm / sa are reused by the next call
}

// Decisions, probabilities and the partial PV of one chunk.
template <int IN, int D, bool PAGED, int GP>
__global__ void __launch_bounds__(256) dec_pv(DecParams p) {
    constexpr bool F8 = IN == BSP_FP8_E4M3;
    constexpr int ES = F8 ? 1 : 2;
    constexpr int LPR = D * ES / 16;
    constexpr int EPL = 16 / ES;
    constexpr int RPW = 64 / LPR;
    int s, g, c, kbase, Lk, nblk, j0, j1;
    if (!dec_item(p, s, g, c, kbase, Lk, nblk, j0, j1)) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int sub = lane % LPR, rw = lane / LPR;
    const int G = p.G;
    __shared__ float sred[4][GP][2];
    __shared__ float sacc[4][GP][D + 1];

    // overall max and the max before this chunk, per head, from the block maxima
    float mall[GP], mpre[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) mall[h] = mpre[h] = -INFINITY;
    for (int j = tid; j < nblk; j += 256) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            if (h < G) {
                const float x = p.M[((int64_t)(g * G + h) * p.n_seqs + s) * p.J_max + j];
                mall[h] = fmaxf(mall[h], x);
                if (j < j0) mpre[h] = fmaxf(mpre[h], x);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            mall[h] = fmaxf(mall[h], __shfl_xor(mall[h], m));
            mpre[h] = fmaxf(mpre[h], __shfl_xor(mpre[h], m));
        }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            sred[w][h][0] = mall[h];
            sred[w][h][1] = mpre[h];
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        mall[h] = fmaxf(fmaxf(sred[0][h][0], sred[1][h][0]), fmaxf(sred[2][h][0], sred[3][h][0]));
        mpre[h] = fmaxf(fmaxf(sred[0][h][1], sred[1][h][1]), fmaxf(sred[2][h][1], sred[3][h][1]));
    }
    float lam_raw = p.lam_raw;
    if (p.lam_seq != nullptr) {
        const float ls = p.lam_seq[s];
        lam_raw = ls == INFINITY ? INFINITY : ls / p.scale;
    }
    const float cl = p.c_log2;
    const bool load_all = (p.flags & BSP_FLAG_LOAD_SKIPPED_V) != 0;
    const bool exp_all = (p.flags & BSP_FLAG_EXP_SKIPPED) != 0;
    const char *vg = (const char *)p.v + (int64_t)g * p.v_sh * ES;
    const int64_t vst = p.v_st * ES;
    const float *Sg = p.S + ((int64_t)g * p.total_k + kbase) * GP;

    // the chunk's decisions, block by block in order, one thread per head
    __shared__ uint8_t skeep[GP][kDecMaxC];
    unsigned long long nskip = 0;
    if (tid < G && tid < GP) {
        const int h = tid;
        float m = -INFINITY;
#pragma unroll
        for (int x = 0; x < GP; ++x) m = x == h ? mpre[x] : m;
        const float *Mh = p.M + ((int64_t)(g * G + h) * p.n_seqs + s) * p.J_max;
        for (int j = j0; j < j1; ++j) {
            const float mj = Mh[j];
            const bool keep = !(m - mj > lam_raw);  // strict: a gap equal to lambda keeps the block
            m = fmaxf(m, mj);
            skeep[h][j - j0] = keep ? 1 : 0;
            if (!keep) {
                ++nskip;
                if (p.bitmap != nullptr)
                    atomicOr(&p.bitmap[((int64_t)(g * G + h) * p.n_seqs + s) * p.W + (j >> 5)], 1u << (j & 31));
            }
        }
    }
    __syncthreads();

    float acc[GP][EPL];
    float lsum[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        lsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
    // the chunk's blocks go round-robin to the 4 waves
    for (int j = j0 + w; j < j1; j += 4) {
        bool keep[GP];  // wave-uniform (read through readfirstlane so that the branches below are scalar)
        bool any = false;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            keep[h] = h < G && __builtin_amdgcn_readfirstlane((int)skeep[h][j - j0]) != 0;
            any = any || keep[h];
        }
        if (!any && !load_all) continue;
        const int kb = j * p.BK;
        const int rows = min(p.BK, Lk - kb);
        for (int r0 = 0; r0 < rows; r0 += RPW * kDecRows) {
            u32x4 xs[kDecRows];
            float sc[kDecRows][GP];
#pragma unroll
            for (int u = 0; u < kDecRows; ++u) {
                const int key = kb + min(r0 + RPW * u + rw, rows - 1);
                xs[u] = *(const u32x4 *)(dec_row<PAGED>(p, vg, vst, s, kbase, key) + 16 * sub);
                // the GP scores of the row in one load
                if constexpr (GP == 1) {
                    sc[u][0] = Sg[key];
                } else if constexpr (GP == 2) {
                    const u32x2 y = *(const u32x2 *)(Sg + (int64_t)key * 2);
                    const uint32_t y0 = y[0], y1 = y[1];
                    sc[u][0] = __builtin_bit_cast(float, y0);
                    sc[u][1] = __builtin_bit_cast(float, y1);
                } else {
#pragma unroll
                    for (int h4 = 0; h4 < GP; h4 += 4) {
                        const f32x4 y = *(const f32x4 *)(Sg + (int64_t)key * GP + h4);
#pragma unroll
                        for (int i = 0; i < 4; ++i) sc[u][h4 + i] = y[i];
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kDecRows; ++u) {
                const bool ok = r0 + RPW * u + rw < rows;
                float vf[EPL];
                widen16<F8>(xs[u], vf);
#pragma unroll
                for (int h = 0; h < GP; ++h) {
                    if (keep[h]) {
                        const float e2 = __builtin_amdgcn_exp2f((sc[u][h] - mall[h]) * cl);
                        const float pe = ok ? e2 : 0.f;  // rows past the block end add nothing
                        lsum[h] += pe;
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pe, vf[e], acc[h][e]);
                    } else if (exp_all && h < G) {
                        // ablation: the exponential of a skipped key, computed and dropped
                        const float pe = __builtin_amdgcn_exp2f((sc[u][h] - mall[h]) * cl);
                        asm volatile("" ::"v"(pe));
                    }
                }
            }
        }
    }
    // partial sums: over the rows of this wave (lanes with the same dims), then over the 4 waves
#pragma unroll
    for (int h = 0; h < GP; ++h) {
#pragma unroll
        for (int m = LPR; m < 64; m <<= 1) {
            lsum[h] += __shfl_xor(lsum[h], m);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], m);
        }
    }
    if (rw == 0) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sacc[w][h][sub * EPL + e] = acc[h][e];
            if (sub == 0) sacc[w][h][D] = lsum[h];
        }
    }
    __syncthreads();
    for (int i = tid; i < G * (D + 1) && i < GP * (D + 1); i += 256) {
        const int h = i / (D + 1), d = i % (D + 1);
        const float x = (sacc[0][h][d] + sacc[1][h][d]) + (sacc[2][h][d] + sacc[3][h][d]);
        p.part[(((int64_t)(g * G + h) * p.n_seqs + s) * p.n_chunks + c) * (D + 1) + d] = x;
    }
    if (tid < G && tid < GP) {
        const unsigned long long vis = (unsigned long long)(j1 - j0);
        if (p.skip_count) atomicAdd(&p.skip_count[g * G + tid], nskip);
        if (p.visited_count) atomicAdd(&p.visited_count[g * G + tid], vis);
        if (p.seq_skip) atomicAdd(&p.seq_skip[s], nskip);
        if (p.seq_visited) atomicAdd(&p.seq_visited[s], vis);
    }
}

// o and lse from the chunk partials, one workgroup per (sequence, query head).
// (A combine by the last chunk's workgroup, behind an arrival counter, needs a
// device-scope fence in every workgroup; on this GPU that writes back the L2
// and made the step slower than a separate launch.)
template <int D>
__global__ void __launch_bounds__(256) dec_combine(DecParams p) {
    const int hq = blockIdx.x % p.Hq, s = blockIdx.x / p.Hq;
    const int kbase = p.cu_k[s];
    const int Lk = p.cu_k[s + 1] - kbase;
    const int nblk = Lk > 0 ? min((Lk + p.BK - 1) / p.BK, p.J_max) : 0;
    if (nblk == 0) return;  // a sequence without keys: nothing written
    dec_combine_head<D>(p, s, hq, nblk);
}

// Zero the bitmap and the counters ahead of the main kernel (a plain fill
// kernel keeps the call free of memset nodes).
__global__ void __launch_bounds__(256) fill_outputs(uint32_t *bitmap, int64_t words, unsigned long long *c0,
                                                    unsigned long long *c1, int n_heads, unsigned long long *c2,
                                                    unsigned long long *c3, int n_seqs) {
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if (bitmap)
        for (int64_t i = i0; i < words; i += stride) bitmap[i] = 0u;
    for (int64_t i = i0; i < n_heads; i += stride) {
        if (c0) c0[i] = 0ull;
        if (c1) c1[i] = 0ull;
    }
    for (int64_t i = i0; i < n_seqs; i += stride) {
        if (c2) c2[i] = 0ull;
        if (c3) c3[i] = 0ull;
    }
}

// ---------------------------------------------------------------------------
// Host side: validation, dispatch, launch.
// ---------------------------------------------------------------------------
thread_local char g_detail[512] = "";

bsp_status_t fail(bsp_status_t st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
bsp_status_t fail(bsp_status_t st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return st;
}

int elem_size(int dtype) { return dtype == BSP_F32 ? 4 : dtype == BSP_BF16 ? 2 : dtype == BSP_FP8_E4M3 ? 1 : 0; }

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

bsp_status_t check_tensor(const char *name, const bsp_tensor_t *x, int heads, int head_dim) {
    if (x == nullptr || x->data == nullptr) return fail(BSP_ERR_INVALID_ARG, "%s: NULL tensor or data", name);
    const int es = elem_size(x->dtype);
    if (es == 0) return fail(BSP_ERR_INVALID_ARG, "%s: unknown dtype %d", name, (int)x->dtype);
    if (!aligned16(x->data)) return fail(BSP_ERR_INVALID_ARG, "%s: data pointer not 16-byte aligned", name);
    const int64_t q = 16 / es;
    if (x->stride_token <= 0 || x->stride_head <= 0 || x->stride_token % q != 0 || x->stride_head % q != 0)
        return fail(BSP_ERR_INVALID_ARG, "%s: strides must be positive multiples of %lld elements", name, (long long)q);
    if (heads > 1 && x->stride_head < head_dim)
        return fail(BSP_ERR_INVALID_ARG, "%s: stride_head %lld < head_dim", name, (long long)x->stride_head);
    return BSP_OK;
}

typedef void (*kernel_fn)(FwdParams);

template <int IN, int D, int BQ, int BK, bool DENSE>
kernel_fn pick_mfma2(bool paged, int hpw) {
    if (hpw == 2) return paged ? fwd_mfma<IN, D, BQ, BK, true, 2, DENSE> : fwd_mfma<IN, D, BQ, BK, false, 2, DENSE>;
    return paged ? fwd_mfma<IN, D, BQ, BK, true, 1, DENSE> : fwd_mfma<IN, D, BQ, BK, false, 1, DENSE>;
}
template <int IN, int D, int BQ, int BK>
kernel_fn pick_mfma(bool paged, int hpw, bool dense) {
    return dense ? pick_mfma2<IN, D, BQ, BK, true>(paged, hpw) : pick_mfma2<IN, D, BQ, BK, false>(paged, hpw);
}

template <int D, int BQ, int BK>
kernel_fn pick_kernel(int dtype, bool paged, int hpw, bool dense) {
    if (dtype == BSP_BF16) return pick_mfma<BSP_BF16, D, BQ, BK>(paged, hpw, dense);
    if (dtype == BSP_FP8_E4M3) {
        if constexpr (D == 128) return pick_mfma<BSP_FP8_E4M3, D, BQ, BK>(paged, hpw, dense);
        return nullptr;  // fp8 kernels are built for head_dim 128 only
    }
    if (dtype == BSP_F32) return paged ? fwd_f32<D, BQ, BK, true> : fwd_f32<D, BQ, BK, false>;
    return nullptr;
}

// Sparse mode for 64-key blocks (any block_q) on the two-head schedule at 128 x 128
// (bf16; fp8 with packed K/V, where that schedule fits the registers).
template <int IN, int D>
kernel_fn key_half_kernel(bool paged) {
    return paged ? fwd_mfma<IN, D, 128, 128, true, 2, false, true> : fwd_mfma<IN, D, 128, 128, false, 2, false, true>;
}
kernel_fn find_key_half_kernel(int dtype, int D, bool paged) {
    if (dtype == BSP_BF16 && D == 128) return key_half_kernel<BSP_BF16, 128>(paged);
    if (dtype == BSP_BF16 && D == 64) return key_half_kernel<BSP_BF16, 64>(paged);
    if (dtype == BSP_FP8_E4M3 && D == 128 && !paged) return fwd_mfma<BSP_FP8_E4M3, 128, 128, 128, false, 2, false, true>;
    return nullptr;
}

// Query heads per workgroup: the bf16 and fp8 kernels pair the query heads of
// a KV head when the group size is even.
int heads_per_workgroup(int dtype, int group) { return (dtype != BSP_F32 && group % 2 == 0) ? 2 : 1; }

kernel_fn find_kernel(int dtype, int D, int BQ, int BK, bool paged, int hpw, bool dense) {
#define BSP_CASE(d, bq, bk) \
    if (D == d && BQ == bq && BK == bk) return pick_kernel<d, bq, bk>(dtype, paged, hpw, dense);
    BSP_CASE(64, 64, 64)
    BSP_CASE(64, 128, 64)
    BSP_CASE(64, 128, 128)
    BSP_CASE(128, 64, 64)
    BSP_CASE(128, 128, 64)
    BSP_CASE(128, 128, 128)
#undef BSP_CASE
    return nullptr;
}

std::mutex g_dev_mu;
int g_dev_ok[64];  // 0 unknown, 1 gfx950, -1 other

bsp_status_t check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(BSP_ERR_DEVICE, "no current HIP device");
    }
    if (dev >= 64) return fail(BSP_ERR_DEVICE, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(BSP_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
        }
        g_dev_ok[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        if (g_dev_ok[dev] < 0) snprintf(g_detail, sizeof(g_detail), "device %d is %s, not gfx950", dev, prop.gcnArchName);
    }
    if (g_dev_ok[dev] < 0) return BSP_ERR_DEVICE;
    return BSP_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- static scratch of bsp_attn_decode_noalloc: the decoding step's workspace
// (scores, block maxima, partial sums) for callers that cannot allocate. Every
// GPU the library runs on holds its own copy until the process ends. Host code
// never passes the array's name to a kernel (in host code it is a host-side
// stand-in): it takes the device address that hipGetSymbolAddress returns,
// once per device with that device current, and passes that.
constexpr int64_t kScratchBytes = BSP_DECODE_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // per device: device address of `scratch`, or NULL until first use

bsp_status_t scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return fail(BSP_ERR_DEVICE, "no current HIP device for the static scratch");
    }
    // the kernels run on the stream's device and take the current device's copy of the array
    if (stream != nullptr) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(BSP_ERR_INVALID_ARG, "cannot query the device of the given stream");
        }
        if (sdev != dev)
            return fail(BSP_ERR_INVALID_ARG, "the stream belongs to device %d but device %d is current", (int)sdev,
                        dev);
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return fail(BSP_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return BSP_OK;
}

// ---- debug validation of device-side descriptors (BSP_DEBUG_VALIDATE)
//
// The sequence bounds and page ids live in device memory, so the normal path
// cannot check them without a synchronisation. With BSP_DEBUG_VALIDATE set
// (to anything but "" or "0") each call first copies them to the host on its
// stream, waits, and checks them, together with the extent of the device
// allocations that hold q, k, v and o; a bad descriptor returns
// BSP_ERR_INVALID_ARG and nothing is launched.
bool debug_validate_enabled() {
    const char *e = getenv("BSP_DEBUG_VALIDATE");
    return e != nullptr && e[0] != '\0' && strcmp(e, "0") != 0;
}

bsp_status_t check_bounds(const char *name, const int32_t *cu, int32_t n, int32_t max_len, int64_t total) {
    if (cu[0] != 0) return fail(BSP_ERR_INVALID_ARG, "%s[0] = %d, must be 0", name, cu[0]);
    for (int32_t s = 0; s < n; ++s) {
        const int64_t len = (int64_t)cu[s + 1] - cu[s];
        if (len < 0) return fail(BSP_ERR_INVALID_ARG, "%s decreases at sequence %d (%d -> %d)", name, s, cu[s], cu[s + 1]);
        if (len > max_len)
            return fail(BSP_ERR_INVALID_ARG, "sequence %d has %lld positions in %s, above the stated maximum %d", s,
                        (long long)len, name, max_len);
    }
    if (total >= 0 && cu[n] != total)
        return fail(BSP_ERR_INVALID_ARG, "%s[n_seqs] = %d, but the call states %lld tokens", name, cu[n], (long long)total);
    return BSP_OK;
}

// Highest element offset + 1 that an access of `rows` token slots of a
// [slots, heads, head_dim] tensor reaches (rows > 0).
int64_t tensor_extent_bytes(const bsp_tensor_t *x, int64_t rows, int heads, int head_dim) {
    const int64_t es = elem_size(x->dtype);
    return ((rows - 1) * x->stride_token + (int64_t)(heads - 1) * x->stride_head + head_dim) * es;
}

// Bytes from x->data to the end of the device allocation holding it (-1: not a device allocation).
int64_t bytes_to_allocation_end(const void *ptr) {
    void *base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (void *)ptr) != hipSuccess || base == nullptr) {
        (void)hipGetLastError();
        return -1;
    }
    return (int64_t)((const char *)base + size - (const char *)ptr);
}

bsp_status_t check_extent(const char *name, const bsp_tensor_t *x, int64_t rows, int heads, int head_dim) {
    if (rows <= 0) return BSP_OK;
    const int64_t avail = bytes_to_allocation_end(x->data);
    if (avail < 0) return fail(BSP_ERR_INVALID_ARG, "%s: data is not inside a device allocation", name);
    const int64_t need = tensor_extent_bytes(x, rows, heads, head_dim);
    if (need > avail)
        return fail(BSP_ERR_INVALID_ARG, "%s: %lld rows need %lld bytes, the allocation holds %lld from the data pointer",
                    name, (long long)rows, (long long)need, (long long)avail);
    return BSP_OK;
}

// Physical pages whose every row a [slots, heads, head_dim] cache tensor holds.
int64_t pages_held(const bsp_tensor_t *x, int page_size, int heads, int head_dim) {
    const int64_t avail = bytes_to_allocation_end(x->data);
    if (avail < 0) return 0;
    const int64_t es = elem_size(x->dtype);
    const int64_t tail = ((int64_t)(heads - 1) * x->stride_head + head_dim - x->stride_token) * es;
    const int64_t per_page = (int64_t)page_size * x->stride_token * es;
    return avail - tail < 0 ? 0 : (avail - tail) / per_page;
}

bsp_status_t copy_to_host(void *dst, const void *src, int64_t bytes, hipStream_t hs, const char *name) {
    if (bytes <= 0) return BSP_OK;
    if (hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToHost, hs) != hipSuccess ||
        hipStreamSynchronize(hs) != hipSuccess) {
        const hipError_t e = hipGetLastError();
        return fail(BSP_ERR_INVALID_ARG, "BSP_DEBUG_VALIDATE: cannot read %s from the device (%s)", name,
                    hipGetErrorString(e));
    }
    return BSP_OK;
}

// Copies the device descriptors of a call to the host and checks them (see above).
// q_rows: query rows (rows of q and o); cu_k NULL: keys = queries.
bsp_status_t validate_call(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v, const bsp_tensor_t *o,
                           const int32_t *cu_q, const int32_t *cu_k, int32_t n_seqs, int32_t max_q, int32_t max_k,
                           int64_t q_rows, int64_t total_q, int64_t total_k, const bsp_block_table_t *bt,
                           const float *lam_seq, int n_heads_q, int n_heads_kv, int head_dim, hipStream_t hs) {
    std::vector<int32_t> hq(cu_q ? n_seqs + 1 : 0), hk(cu_k ? n_seqs + 1 : 0);
    std::vector<int32_t> table(bt ? (size_t)n_seqs * bt->max_pages_per_seq : 0);
    std::vector<float> lams(lam_seq ? n_seqs : 0);
    bsp_status_t st;
    if (cu_q && (st = copy_to_host(hq.data(), cu_q, 4 * (int64_t)hq.size(), hs, "cu_seqlens")) != BSP_OK) return st;
    if (cu_k && (st = copy_to_host(hk.data(), cu_k, 4 * (int64_t)hk.size(), hs, "cu_seqlens_k")) != BSP_OK) return st;
    if (bt && (st = copy_to_host(table.data(), bt->table, 4 * (int64_t)table.size(), hs, "the block table")) != BSP_OK)
        return st;
    if (lam_seq && (st = copy_to_host(lams.data(), lam_seq, 4 * (int64_t)lams.size(), hs, "lambda_per_seq")) != BSP_OK)
        return st;
    int64_t n_pages = 0;
    if (bt) {
        const int64_t pk = pages_held(k, bt->page_size, n_heads_kv, head_dim);
        const int64_t pv = pages_held(v, bt->page_size, n_heads_kv, head_dim);
        n_pages = pk < pv ? pk : pv;
        if (n_pages <= 0) return fail(BSP_ERR_INVALID_ARG, "the paged k/v tensors hold no whole page");
    }
    st = bsp_validate_host(cu_q ? hq.data() : nullptr, cu_k ? hk.data() : nullptr, n_seqs, max_q, max_k, total_q,
                           bt ? -1 : total_k, bt ? table.data() : nullptr, bt ? bt->max_pages_per_seq : 0,
                           bt ? bt->page_size : 0, n_pages);
    if (st != BSP_OK) return st;
    for (int32_t s = 0; s < (int32_t)lams.size(); ++s)
        if (std::isnan(lams[s]) || lams[s] < 0.f)
            return fail(BSP_ERR_INVALID_ARG, "lambda_per_seq[%d] = %g: must be >= 0 or +inf", s, lams[s]);
    if ((st = check_extent("q", q, q_rows, n_heads_q, head_dim)) != BSP_OK) return st;
    if ((st = check_extent("o", o, q_rows, n_heads_q, head_dim)) != BSP_OK) return st;
    if (!bt) {
        if ((st = check_extent("k", k, total_k, n_heads_kv, head_dim)) != BSP_OK) return st;
        if ((st = check_extent("v", v, total_k, n_heads_kv, head_dim)) != BSP_OK) return st;
    }
    return BSP_OK;
}

// ---- decoding step: instances, chunking and workspace layout
typedef void (*dec_fn)(DecParams);
struct DecKernels {
    dec_fn scores, pv, combine;
};
template <int IN, int D, bool PAGED, int GP>
DecKernels dec_kernels() {
    return {dec_scores<IN, D, PAGED, GP>, dec_pv<IN, D, PAGED, GP>, dec_combine<D>};
}
template <int IN, int D, bool PAGED>
DecKernels dec_by_group(int G) {
    if (G <= 1) return dec_kernels<IN, D, PAGED, 1>();
    if (G <= 2) return dec_kernels<IN, D, PAGED, 2>();
    if (G <= 4) return dec_kernels<IN, D, PAGED, 4>();
    return dec_kernels<IN, D, PAGED, 8>();
}
bool find_dec(int dtype, int D, bool paged, int G, DecKernels &out) {
    if (G > 8) return false;
    if (dtype == BSP_BF16 && D == 128) out = paged ? dec_by_group<BSP_BF16, 128, true>(G) : dec_by_group<BSP_BF16, 128, false>(G);
    else if (dtype == BSP_BF16 && D == 64) out = paged ? dec_by_group<BSP_BF16, 64, true>(G) : dec_by_group<BSP_BF16, 64, false>(G);
    else if (dtype == BSP_FP8_E4M3 && D == 128) out = paged ? dec_by_group<BSP_FP8_E4M3, 128, true>(G) : dec_by_group<BSP_FP8_E4M3, 128, false>(G);
    else return false;
    return true;
}

// Key blocks per chunk: about 4096 (sequence, KV head, chunk) work items.
struct DecLayout {
    int64_t J_max, C, n_chunks, s_off, m_off, part_off, bytes;
};
DecLayout dec_layout(int n_heads_q, int n_heads_kv, int n_seqs, int64_t total_k, int max_k, int head_dim, int block_k) {
    DecLayout L;
    L.J_max = cdiv(max_k, block_k);
    const int64_t units = (int64_t)n_seqs * n_heads_kv * L.J_max;
    // about 4096 work items; chunks of whole multiples of 4 blocks (one per wave), at most kDecMaxC
    L.C = units > 4096 * 4 ? 4 * cdiv(units, 4096 * 4) : 4;
    if (L.C > kDecMaxC) L.C = kDecMaxC;
    L.n_chunks = L.J_max > 0 ? cdiv(L.J_max, L.C) : 0;
    auto up = [](int64_t x) { return (x + 255) & ~(int64_t)255; };
    L.s_off = 0;
    const int G = n_heads_q / n_heads_kv;
    const int GP = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
    L.m_off = up((int64_t)n_heads_kv * total_k * GP * 4);
    L.part_off = L.m_off + up((int64_t)n_heads_q * n_seqs * L.J_max * 4);
    L.bytes = L.part_off + up((int64_t)n_heads_q * n_seqs * L.n_chunks * (head_dim + 1) * 4);
    return L;
}

}  // namespace

extern "C" {

int bsp_version(void) { return 200; }

const char *bsp_status_string(int status) {
    switch (status) {
        case BSP_OK: return "ok";
        case BSP_ERR_INVALID_ARG: return "invalid argument";
        case BSP_ERR_UNSUPPORTED: return "unsupported configuration";
        case BSP_ERR_HIP: return "HIP error";
        case BSP_ERR_DEVICE: return "device error";
        default: return "unknown status";
    }
}

const char *bsp_last_error_detail(void) { return g_detail; }

int64_t bsp_skip_bitmap_words_kv(int n_heads_q, int n_seqs, int max_seqlen_q, int max_seqlen_k, int block_q,
                                 int block_k) {
    if (n_heads_q <= 0 || n_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || block_q <= 0 || block_k <= 0)
        return 0;
    const int64_t T = cdiv(max_seqlen_q, block_q);
    const int64_t J = cdiv(max_seqlen_k, block_k);
    const int64_t W = cdiv(J, 32);
    return (int64_t)n_heads_q * n_seqs * T * W;
}

bsp_status_t bsp_validate_host(const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t n_seqs,
                               int32_t max_seqlen_q, int32_t max_seqlen_k, int64_t total_q, int64_t total_k,
                               const int32_t *block_table, int32_t max_pages_per_seq, int32_t page_size,
                               int64_t n_pages) {
    g_detail[0] = '\0';
    if (n_seqs < 0 || cu_seqlens_q == nullptr) return fail(BSP_ERR_INVALID_ARG, "no sequence descriptor");
    bsp_status_t st;
    if ((st = check_bounds("cu_seqlens", cu_seqlens_q, n_seqs, max_seqlen_q, total_q)) != BSP_OK) return st;
    const int32_t *cu_k = cu_seqlens_k ? cu_seqlens_k : cu_seqlens_q;
    if (cu_seqlens_k != nullptr) {
        if ((st = check_bounds("cu_seqlens_k", cu_k, n_seqs, max_seqlen_k, total_k)) != BSP_OK) return st;
        for (int32_t s = 0; s < n_seqs; ++s)
            if (cu_k[s + 1] - cu_k[s] < cu_seqlens_q[s + 1] - cu_seqlens_q[s])
                return fail(BSP_ERR_INVALID_ARG, "sequence %d has %d queries but only %d keys", s,
                            cu_seqlens_q[s + 1] - cu_seqlens_q[s], cu_k[s + 1] - cu_k[s]);
    }
    if (block_table != nullptr) {
        if (page_size <= 0 || max_pages_per_seq < 0) return fail(BSP_ERR_INVALID_ARG, "bad page geometry");
        for (int32_t s = 0; s < n_seqs; ++s) {
            const int64_t pages = cdiv((int64_t)cu_k[s + 1] - cu_k[s], page_size);
            if (pages > max_pages_per_seq)
                return fail(BSP_ERR_INVALID_ARG, "sequence %d needs %lld pages, the table row holds %d", s,
                            (long long)pages, max_pages_per_seq);
            for (int64_t pg = 0; pg < pages; ++pg) {
                const int32_t id = block_table[(int64_t)s * max_pages_per_seq + pg];
                if (id < 0 || (n_pages > 0 && id >= n_pages))
                    return fail(BSP_ERR_INVALID_ARG, "block_table[%d][%lld] = %d is outside the %lld pages of the cache",
                                s, (long long)pg, id, (long long)n_pages);
            }
        }
    }
    return BSP_OK;
}

int64_t bsp_skip_bitmap_words(int n_heads_q, int n_seqs, int max_seqlen, int block_q, int block_k) {
    return bsp_skip_bitmap_words_kv(n_heads_q, n_seqs, max_seqlen, max_seqlen, block_q, block_k);
}

bsp_status_t bsp_attn_fwd(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v, bsp_tensor_t *o,
                          float *lse, const bsp_seqs_t *seqs, const bsp_block_table_t *bt, int n_heads_q,
                          int n_heads_kv, int head_dim, int block_q, int block_k, float lambda,
                          bsp_skip_out_t *skip_out, void *stream) {
    return bsp_attn_fwd_ex(q, k, v, o, lse, seqs, bt, n_heads_q, n_heads_kv, head_dim, block_q, block_k, lambda,
                           skip_out, stream, nullptr);
}

bsp_status_t bsp_attn_fwd_ex(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v, bsp_tensor_t *o,
                             float *lse, const bsp_seqs_t *seqs, const bsp_block_table_t *bt, int n_heads_q,
                             int n_heads_kv, int head_dim, int block_q, int block_k, float lambda,
                             bsp_skip_out_t *skip_out, void *stream, const bsp_fwd_options_t *opts) {
    g_detail[0] = '\0';
    bsp_fwd_options_t none;
    memset(&none, 0, sizeof(none));
    if (opts == nullptr) opts = &none;
    if ((opts->flags & ~(BSP_FLAG_LOAD_SKIPPED_V | BSP_FLAG_EXP_SKIPPED)) != 0)
        return fail(BSP_ERR_INVALID_ARG, "unknown option flags 0x%x", opts->flags);
    const bool chunked = opts->cu_seqlens_k != nullptr;
    if (chunked && (opts->max_seqlen_k < 0 || ((uintptr_t)opts->cu_seqlens_k & 3u) != 0))
        return fail(BSP_ERR_INVALID_ARG, "cu_seqlens_k needs max_seqlen_k >= 0 and 4-byte alignment");
    if (opts->lambda_per_seq != nullptr && ((uintptr_t)opts->lambda_per_seq & 3u) != 0)
        return fail(BSP_ERR_INVALID_ARG, "lambda_per_seq not 4-byte aligned");
    if (((uintptr_t)opts->skip_count_per_seq & 7u) != 0 || ((uintptr_t)opts->visited_count_per_seq & 7u) != 0)
        return fail(BSP_ERR_INVALID_ARG, "per-sequence counts not 8-byte aligned");
    // ---------------- argument checks (host only, before any HIP call)
    if (n_heads_q <= 0 || n_heads_kv <= 0 || n_heads_q % n_heads_kv != 0)
        return fail(BSP_ERR_INVALID_ARG, "n_heads_q (%d) must be a positive multiple of n_heads_kv (%d)", n_heads_q,
                    n_heads_kv);
    if (head_dim <= 0) return fail(BSP_ERR_INVALID_ARG, "head_dim must be positive");
    if (isnan(lambda) || lambda < 0.f) return fail(BSP_ERR_INVALID_ARG, "lambda must be >= 0 or +inf (got %g)", lambda);
    if (block_q <= 0 || block_k <= 0) return fail(BSP_ERR_INVALID_ARG, "block sizes must be positive");
    bsp_status_t st;
    if ((st = check_tensor("q", q, n_heads_q, head_dim)) != BSP_OK) return st;
    if ((st = check_tensor("k", k, n_heads_kv, head_dim)) != BSP_OK) return st;
    if ((st = check_tensor("v", v, n_heads_kv, head_dim)) != BSP_OK) return st;
    if ((st = check_tensor("o", o, n_heads_q, head_dim)) != BSP_OK) return st;
    if (k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(BSP_ERR_INVALID_ARG, "q, k and v must share one dtype");
    const int want_o = q->dtype == BSP_F32 ? BSP_F32 : BSP_BF16;
    if (o->dtype != want_o) return fail(BSP_ERR_INVALID_ARG, "o must be %s for this input dtype", want_o == BSP_F32 ? "f32" : "bf16");
    if (q->dtype == BSP_FP8_E4M3 && (!q->scale || !k->scale || !v->scale))
        return fail(BSP_ERR_INVALID_ARG, "fp8 inputs need per-head scales on q, k and v");
    if (seqs == nullptr || seqs->cu_seqlens == nullptr) return fail(BSP_ERR_INVALID_ARG, "cu_seqlens is required");
    if (seqs->n_seqs < 0 || seqs->max_seqlen < 0 || seqs->total_tokens < 0)
        return fail(BSP_ERR_INVALID_ARG, "negative sequence sizes");
    if (((uintptr_t)seqs->cu_seqlens & 3u) != 0) return fail(BSP_ERR_INVALID_ARG, "cu_seqlens not 4-byte aligned");
    if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return fail(BSP_ERR_INVALID_ARG, "lse not 4-byte aligned");
    const bool paged = bt != nullptr;
    int page_shift = 0;
    if (paged) {
        if (bt->table == nullptr) return fail(BSP_ERR_INVALID_ARG, "block_table->table is NULL");
        const int ps = bt->page_size;
        if (ps <= 0 || (ps & (ps - 1)) != 0) return fail(BSP_ERR_INVALID_ARG, "page_size must be a power of two");
        if (block_k % ps != 0 && ps % block_k != 0)
            return fail(BSP_ERR_INVALID_ARG, "block_k (%d) and page_size (%d) must divide one another", block_k, ps);
        while ((1 << page_shift) < ps) ++page_shift;
    }
    const int max_k = chunked ? opts->max_seqlen_k : seqs->max_seqlen;  // key positions per sequence
    if (paged && (int64_t)bt->max_pages_per_seq * bt->page_size < max_k)
        return fail(BSP_ERR_INVALID_ARG, "max_pages_per_seq * page_size < max_seqlen%s", chunked ? "_k" : "");
    const int64_t T_max = cdiv(seqs->max_seqlen, block_q);
    const int64_t J_max = cdiv(max_k, block_k);
    const int64_t W = cdiv(J_max, 32);
    uint32_t *bitmap = skip_out ? skip_out->bitmap : nullptr;
    const int64_t words = bsp_skip_bitmap_words_kv(n_heads_q, seqs->n_seqs, seqs->max_seqlen, max_k, block_q, block_k);
    if (bitmap != nullptr) {
        if (((uintptr_t)bitmap & 3u) != 0) return fail(BSP_ERR_INVALID_ARG, "bitmap not 4-byte aligned");
        if (skip_out->bitmap_words < words)
            return fail(BSP_ERR_INVALID_ARG, "bitmap holds %lld words, %lld needed", (long long)skip_out->bitmap_words,
                        (long long)words);
    }
    const int hpw = heads_per_workgroup(q->dtype, n_heads_q / n_heads_kv);
    // dense-mode kernel: lambda = +inf for every sequence (no vote, nothing to ablate)
    const bool dense = isinf(lambda) && opts->lambda_per_seq == nullptr;
    kernel_fn fn = find_kernel(q->dtype, head_dim, block_q, block_k, paged, hpw, dense);
    if (fn == nullptr)
        return fail(BSP_ERR_UNSUPPORTED, "no kernel for dtype %d, head_dim %d, block_q %d, block_k %d", (int)q->dtype,
                    head_dim, block_q, block_k);
    // Dense mode decides nothing, so O and LSE do not depend on the block sizes (up to
    // rounding order) and the bitmap stays zero: run the 128 x 128 instance (the
    // fastest schedule) and count visited blocks in the caller's units.
    int kbq = block_q, kbk = block_k;
    if (dense && q->dtype != BSP_F32 && (block_q != 128 || block_k != 128) && 128 % block_q == 0) {
        kernel_fn f128 = find_kernel(q->dtype, head_dim, 128, 128, paged, hpw, true);
        if (f128 != nullptr) {
            fn = f128;
            kbq = kbk = 128;
        }
    }
    // Sparse mode at 64-row tiles or 64-key blocks: the 128 x 128 instance runs the
    // two-head ping-pong schedule, each 64-row half of its tile votes on its own
    // and each 64-key half of its block is decided on its own, so the decisions,
    // the bitmap and the counts stay those of the caller's blocks.
    int half_vote = 0;
    if (!dense && block_k == 64 && hpw == 2) {
        kernel_fn fkh = find_key_half_kernel(q->dtype, head_dim, paged);
        if (fkh != nullptr) {
            fn = fkh;
            half_vote = block_q == 64 ? 1 : 0;
            kbq = kbk = 128;
        }
    }
    // K/V copies address rows with 32-bit byte offsets from the first row of a block or a page.
    {
        const int64_t es = elem_size(q->dtype);
        const int64_t rows = paged && bt->page_size > kbk ? bt->page_size : kbk;
        if (rows * k->stride_token * es >= (1LL << 31) || rows * v->stride_token * es >= (1LL << 31))
            return fail(BSP_ERR_UNSUPPORTED, "k/v token stride too large (max(block_k, page_size) * stride must stay below 2 GiB)");
    }
    const int64_t T_launch = cdiv(seqs->max_seqlen, kbq);
    const int64_t grid64 = T_launch * (int64_t)seqs->n_seqs * (n_heads_q / hpw);
    if (grid64 > 0x7fffffffLL) return fail(BSP_ERR_INVALID_ARG, "too many work items");

    // ---------------- device
    if ((st = check_device()) != BSP_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    if (debug_validate_enabled()) {
        const int64_t total_k = chunked ? -1 : seqs->total_tokens;  // with cu_seqlens_k: cu_k[n] itself
        st = validate_call(q, k, v, o, seqs->cu_seqlens, opts->cu_seqlens_k, seqs->n_seqs, seqs->max_seqlen, max_k,
                           seqs->total_tokens, seqs->total_tokens, total_k, bt, opts->lambda_per_seq, n_heads_q,
                           n_heads_kv, head_dim, hs);
        if (st != BSP_OK) return st;
        if (chunked && !paged) {  // the packed k/v rows the keys address
            int32_t last = 0;
            if ((st = copy_to_host(&last, opts->cu_seqlens_k + seqs->n_seqs, 4, hs, "cu_seqlens_k")) != BSP_OK) return st;
            if ((st = check_extent("k", k, last, n_heads_kv, head_dim)) != BSP_OK) return st;
            if ((st = check_extent("v", v, last, n_heads_kv, head_dim)) != BSP_OK) return st;
        }
    }
    unsigned long long *c0 = skip_out ? skip_out->skip_count : nullptr;
    unsigned long long *c1 = skip_out ? skip_out->visited_count : nullptr;
    unsigned long long *c2 = opts->skip_count_per_seq;
    unsigned long long *c3 = opts->visited_count_per_seq;
    if (bitmap != nullptr || c0 != nullptr || c1 != nullptr || c2 != nullptr || c3 != nullptr) {
        int64_t work = words > n_heads_q ? words : n_heads_q;
        if (work < seqs->n_seqs) work = seqs->n_seqs;
        const int blocks = (int)(cdiv(work, 256) < 1024 ? cdiv(work, 256) : 1024);
        hipLaunchKernelGGL(fill_outputs, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, hs, bitmap, words, c0, c1,
                           n_heads_q, c2, c3, seqs->n_seqs);
    }
    if (grid64 > 0) {
        FwdParams p;
        memset(&p, 0, sizeof(p));
        p.q = q->data;
        p.k = k->data;
        p.v = v->data;
        p.o = o->data;
        p.lse = lse;
        p.q_st = q->stride_token;
        p.q_sh = q->stride_head;
        p.k_st = k->stride_token;
        p.k_sh = k->stride_head;
        p.v_st = v->stride_token;
        p.v_sh = v->stride_head;
        p.o_st = o->stride_token;
        p.o_sh = o->stride_head;
        p.lse_sh = seqs->total_tokens;
        p.cu = seqs->cu_seqlens;
        p.table = paged ? bt->table : nullptr;
        p.max_pages = paged ? bt->max_pages_per_seq : 0;
        p.page_shift = page_shift;
        p.bitmap = bitmap;
        p.skip_count = c0;
        p.visited_count = c1;
        p.n_seqs = seqs->n_seqs;
        p.T_max = (int32_t)T_launch;  // tiles of the launched kernel
        p.T_bm = (int32_t)T_max;      // bitmap tiles: the caller's (dense mode writes no bitmap)
        p.half_vote = half_vote;
        p.W = (int32_t)W;
        p.Hq = n_heads_q;
        p.Hkv = n_heads_kv;
        p.G = n_heads_q / n_heads_kv;
        p.xcd_mode = (n_heads_kv % 8 == 0) ? 1 : 0;
        p.hpw = hpw;
        const double scale = 1.0 / sqrt((double)head_dim);
        p.c_log2 = (float)(scale * 1.4426950408889634);
        p.lam_raw = isinf(lambda) ? INFINITY : (float)((double)lambda / scale);
        p.q_scale = q->scale;
        p.k_scale = k->scale;
        p.v_scale = v->scale;
        p.scale = (float)scale;
        p.lam = lambda;
        p.cu_k = opts->cu_seqlens_k;
        p.lam_seq = opts->lambda_per_seq;
        p.seq_skip = c2;
        p.seq_visited = c3;
        p.flags = opts->flags;
        // counts in the caller's blocks when the launched tile differs from them
        p.acct_bq = (kbq != block_q || kbk != block_k) ? block_q : 0;
        p.acct_bk = (kbq != block_q || kbk != block_k) ? block_k : 0;
        hipLaunchKernelGGL(fn, dim3((unsigned)grid64), dim3(kbq * 2 * hpw), 0, hs, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return BSP_OK;
}

int64_t bsp_decode_workspace_bytes(int n_heads_q, int n_heads_kv, int n_seqs, int64_t total_k, int max_seqlen_k,
                                   int head_dim, int block_k) {
    if (n_heads_q <= 0 || n_heads_kv <= 0 || n_seqs < 0 || total_k < 0 || max_seqlen_k < 0 || head_dim <= 0 ||
        block_k <= 0)
        return -1;
    return dec_layout(n_heads_q, n_heads_kv, n_seqs, total_k, max_seqlen_k, head_dim, block_k).bytes;
}

// bsp_attn_decode (caller's workspace) and bsp_attn_decode_noalloc (the static
// scratch array of the current device) share everything but where the
// workspace comes from.
static bsp_status_t decode_call(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v, bsp_tensor_t *o,
                                float *lse, const bsp_seqs_t *seqs_k, const bsp_block_table_t *bt, int n_heads_q,
                                int n_heads_kv, int head_dim, int block_k, float lambda, bsp_skip_out_t *skip_out,
                                void *stream, const bsp_decode_options_t *opts, void *workspace,
                                int64_t workspace_bytes, bool use_scratch) {
    g_detail[0] = '\0';
    bsp_decode_options_t none;
    memset(&none, 0, sizeof(none));
    if (opts == nullptr) opts = &none;
    if ((opts->flags & ~(BSP_FLAG_LOAD_SKIPPED_V | BSP_FLAG_EXP_SKIPPED)) != 0)
        return fail(BSP_ERR_INVALID_ARG, "unknown option flags 0x%x", opts->flags);
    if (opts->lambda_per_seq != nullptr && ((uintptr_t)opts->lambda_per_seq & 3u) != 0)
        return fail(BSP_ERR_INVALID_ARG, "lambda_per_seq not 4-byte aligned");
    if (((uintptr_t)opts->skip_count_per_seq & 7u) != 0 || ((uintptr_t)opts->visited_count_per_seq & 7u) != 0)
        return fail(BSP_ERR_INVALID_ARG, "per-sequence counts not 8-byte aligned");
    if (n_heads_q <= 0 || n_heads_kv <= 0 || n_heads_q % n_heads_kv != 0)
        return fail(BSP_ERR_INVALID_ARG, "n_heads_q (%d) must be a positive multiple of n_heads_kv (%d)", n_heads_q,
                    n_heads_kv);
    if (head_dim <= 0) return fail(BSP_ERR_INVALID_ARG, "head_dim must be positive");
    if (isnan(lambda) || lambda < 0.f) return fail(BSP_ERR_INVALID_ARG, "lambda must be >= 0 or +inf (got %g)", lambda);
    if (block_k <= 0) return fail(BSP_ERR_INVALID_ARG, "block_k must be positive");
    bsp_status_t st;
    if ((st = check_tensor("q", q, n_heads_q, head_dim)) != BSP_OK) return st;
    if ((st = check_tensor("k", k, n_heads_kv, head_dim)) != BSP_OK) return st;
    if ((st = check_tensor("v", v, n_heads_kv, head_dim)) != BSP_OK) return st;
    if ((st = check_tensor("o", o, n_heads_q, head_dim)) != BSP_OK) return st;
    if (k->dtype != q->dtype || v->dtype != q->dtype)
        return fail(BSP_ERR_INVALID_ARG, "q, k and v must share one dtype");
    if (q->dtype == BSP_F32) return fail(BSP_ERR_UNSUPPORTED, "decoding supports bf16 and fp8 e4m3 inputs");
    if (o->dtype != BSP_BF16) return fail(BSP_ERR_INVALID_ARG, "o must be bf16");
    if (q->dtype == BSP_FP8_E4M3 && (!q->scale || !k->scale || !v->scale))
        return fail(BSP_ERR_INVALID_ARG, "fp8 inputs need per-head scales on q, k and v");
    if (seqs_k == nullptr || seqs_k->cu_seqlens == nullptr) return fail(BSP_ERR_INVALID_ARG, "seqs_k->cu_seqlens is required");
    if (seqs_k->n_seqs < 0 || seqs_k->max_seqlen < 0 || seqs_k->total_tokens < 0)
        return fail(BSP_ERR_INVALID_ARG, "negative sequence sizes");
    if (((uintptr_t)seqs_k->cu_seqlens & 3u) != 0) return fail(BSP_ERR_INVALID_ARG, "cu_seqlens not 4-byte aligned");
    if (lse != nullptr && ((uintptr_t)lse & 3u) != 0) return fail(BSP_ERR_INVALID_ARG, "lse not 4-byte aligned");
    const bool paged = bt != nullptr;
    int page_shift = 0;
    if (paged) {
        if (bt->table == nullptr) return fail(BSP_ERR_INVALID_ARG, "block_table->table is NULL");
        const int ps = bt->page_size;
        if (ps <= 0 || (ps & (ps - 1)) != 0) return fail(BSP_ERR_INVALID_ARG, "page_size must be a power of two");
        if ((int64_t)bt->max_pages_per_seq * ps < seqs_k->max_seqlen)
            return fail(BSP_ERR_INVALID_ARG, "max_pages_per_seq * page_size < max_seqlen");
        while ((1 << page_shift) < ps) ++page_shift;
    }
    const int G = n_heads_q / n_heads_kv;
    DecKernels kern;
    if (!find_dec(q->dtype, head_dim, paged, G, kern))
        return fail(BSP_ERR_UNSUPPORTED, "no decode kernel for dtype %d, head_dim %d, %d query heads per KV head",
                    (int)q->dtype, head_dim, G);
    const int n_seqs = seqs_k->n_seqs;
    const DecLayout L = dec_layout(n_heads_q, n_heads_kv, n_seqs, seqs_k->total_tokens, seqs_k->max_seqlen, head_dim,
                                   block_k);
    if (use_scratch) {
        if (L.bytes > kScratchBytes)
            return fail(BSP_ERR_INVALID_ARG,
                        "the call needs %lld bytes of workspace, above the %lld-byte static scratch of "
                        "bsp_attn_decode_noalloc (BSP_DECODE_SCRATCH_BYTES); pass a workspace to bsp_attn_decode",
                        (long long)L.bytes, (long long)kScratchBytes);
    } else if (workspace == nullptr || workspace_bytes < L.bytes || ((uintptr_t)workspace & 255u) != 0) {
        return fail(BSP_ERR_INVALID_ARG, "workspace needs %lld bytes, 256-byte aligned (got %lld)", (long long)L.bytes,
                    (long long)workspace_bytes);
    }
    uint32_t *bitmap = skip_out ? skip_out->bitmap : nullptr;
    const int64_t words = bsp_skip_bitmap_words_kv(n_heads_q, n_seqs, 1, seqs_k->max_seqlen, 1, block_k);
    if (bitmap != nullptr) {
        if (((uintptr_t)bitmap & 3u) != 0) return fail(BSP_ERR_INVALID_ARG, "bitmap not 4-byte aligned");
        if (skip_out->bitmap_words < words)
            return fail(BSP_ERR_INVALID_ARG, "bitmap holds %lld words, %lld needed", (long long)skip_out->bitmap_words,
                        (long long)words);
    }
    const int64_t grid = (int64_t)n_seqs * n_heads_kv * L.n_chunks;
    if (grid > 0x7fffffffLL || (int64_t)n_seqs * n_heads_q > 0x7fffffffLL)
        return fail(BSP_ERR_INVALID_ARG, "too many work items");

    if ((st = check_device()) != BSP_OK) return st;
    hipStream_t hs = (hipStream_t)stream;
    if (use_scratch && (st = scratch_address(hs, &workspace)) != BSP_OK) return st;
    if (debug_validate_enabled()) {
        // the keys as seqs_k states them; one query row per sequence (rows of q and o)
        st = validate_call(q, k, v, o, seqs_k->cu_seqlens, nullptr, n_seqs, seqs_k->max_seqlen, seqs_k->max_seqlen, 0,
                           seqs_k->total_tokens, seqs_k->total_tokens, bt, opts->lambda_per_seq, n_heads_q,
                           n_heads_kv, head_dim, hs);
        if (st != BSP_OK) return st;
        if ((st = check_extent("q", q, n_seqs, n_heads_q, head_dim)) != BSP_OK) return st;
        if ((st = check_extent("o", o, n_seqs, n_heads_q, head_dim)) != BSP_OK) return st;
    }
    unsigned long long *c0 = skip_out ? skip_out->skip_count : nullptr;
    unsigned long long *c1 = skip_out ? skip_out->visited_count : nullptr;
    unsigned long long *c2 = opts->skip_count_per_seq;
    unsigned long long *c3 = opts->visited_count_per_seq;
    // (with work to do, dec_scores zeroes the bitmap and the counts itself)
    if (grid == 0 && (bitmap != nullptr || c0 != nullptr || c1 != nullptr || c2 != nullptr || c3 != nullptr)) {
        int64_t work = words > n_heads_q ? words : n_heads_q;
        if (work < n_seqs) work = n_seqs;
        const int blocks = (int)(cdiv(work, 256) < 1024 ? cdiv(work, 256) : 1024);
        hipLaunchKernelGGL(fill_outputs, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, hs, bitmap, words, c0, c1,
                           n_heads_q, c2, c3, n_seqs);
    }
    if (grid > 0) {
        DecParams p;
        memset(&p, 0, sizeof(p));
        p.q = q->data;
        p.k = k->data;
        p.v = v->data;
        p.o = o->data;
        p.lse = lse;
        p.q_st = q->stride_token;
        p.q_sh = q->stride_head;
        p.k_st = k->stride_token;
        p.k_sh = k->stride_head;
        p.v_st = v->stride_token;
        p.v_sh = v->stride_head;
        p.o_st = o->stride_token;
        p.o_sh = o->stride_head;
        p.lse_sh = n_seqs;
        p.total_k = seqs_k->total_tokens;
        p.cu_k = seqs_k->cu_seqlens;
        p.table = paged ? bt->table : nullptr;
        p.max_pages = paged ? bt->max_pages_per_seq : 0;
        p.page_shift = page_shift;
        p.bitmap = bitmap;
        p.skip_count = c0;
        p.visited_count = c1;
        p.seq_skip = c2;
        p.seq_visited = c3;
        p.n_seqs = n_seqs;
        p.W = (int32_t)cdiv(L.J_max, 32);
        p.J_max = (int32_t)L.J_max;
        p.n_chunks = (int32_t)L.n_chunks;
        p.C = (int32_t)L.C;
        p.BK = block_k;
        p.Hq = n_heads_q;
        p.Hkv = n_heads_kv;
        p.G = G;
        const double scale = 1.0 / sqrt((double)head_dim);
        p.scale = (float)scale;
        p.c_log2 = (float)(scale * 1.4426950408889634);
        p.lam_raw = isinf(lambda) ? INFINITY : (float)((double)lambda / scale);
        p.lam_seq = opts->lambda_per_seq;
        p.q_scale = q->scale;
        p.k_scale = k->scale;
        p.v_scale = q->dtype == BSP_FP8_E4M3 ? v->scale : nullptr;
        p.flags = opts->flags;
        char *ws = (char *)workspace;
        p.S = (float *)(ws + L.s_off);
        p.M = (float *)(ws + L.m_off);
        p.part = (float *)(ws + L.part_off);
        hipLaunchKernelGGL(kern.scores, dim3((unsigned)grid), dim3(256), 0, hs, p);
        hipLaunchKernelGGL(kern.pv, dim3((unsigned)grid), dim3(256), 0, hs, p);
        hipLaunchKernelGGL(kern.combine, dim3((unsigned)((int64_t)n_seqs * n_heads_q)), dim3(256), 0, hs, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(BSP_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    return BSP_OK;
}

bsp_status_t bsp_attn_decode(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v, bsp_tensor_t *o,
                             float *lse, const bsp_seqs_t *seqs_k, const bsp_block_table_t *bt, int n_heads_q,
                             int n_heads_kv, int head_dim, int block_k, float lambda, bsp_skip_out_t *skip_out,
                             void *stream, const bsp_decode_options_t *opts, void *workspace,
                             int64_t workspace_bytes) {
    return decode_call(q, k, v, o, lse, seqs_k, bt, n_heads_q, n_heads_kv, head_dim, block_k, lambda, skip_out, stream,
                       opts, workspace, workspace_bytes, false);
}

bsp_status_t bsp_attn_decode_noalloc(const bsp_tensor_t *q, const bsp_tensor_t *k, const bsp_tensor_t *v,
                                     bsp_tensor_t *o, float *lse, const bsp_seqs_t *seqs_k,
                                     const bsp_block_table_t *bt, int n_heads_q, int n_heads_kv, int head_dim,
                                     int block_k, float lambda, bsp_skip_out_t *skip_out, void *stream,
                                     const bsp_decode_options_t *opts) {
    return decode_call(q, k, v, o, lse, seqs_k, bt, n_heads_q, n_heads_kv, head_dim, block_k, lambda, skip_out, stream,
                       opts, nullptr, 0, true);
}

}  // extern "C"
