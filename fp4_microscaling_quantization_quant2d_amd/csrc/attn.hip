// Fused attention with MXFP8 queries and keys, forward and backward, for
// gfx950.  "Stable FP4 Training via Transposition-Invariant Block
// Quantization", Sec. 3.2 "MXFP8 Attention" and Fig. 3: Q and K enter the
// score product in MXFP8 (E4M3, one E8M0 scale per 1x32 group along the head
// dimension); the attention around it is standard scaled dot-product
// attention.  The score matrix S never leaves the chip.
//
// Products.  An E4M3 code times its E8M0 scale is exactly a bf16 value (4
// significant bits), so Q and K are converted to bf16 with the scale folded
// in and every score product q_d * k_d is formed exactly by the bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) and summed in fp32.  The probabilities P (and
// in the backward dS) are rounded to bf16 to multiply V (dO, Q, K), which are
// bf16 already; accumulation is fp32 throughout.
//
// Orientation.  The forward computes S^T = K Q^T per 32-key x 32-query
// block, so a lane holds one query's scores in registers (keys
// 8(r/4) + 4h + r%4 of register r, h = lane/32) and the softmax reductions
// are register reductions plus one exchange with lane l ^ 32.  The same
// registers are the B operand of O^T += V^T P^T once the MFMA's contraction
// index (h, p) is mapped to key 8(2t + p/4) + 4h + p%4 of each 16-key step t
// -- a permutation of the keys that the A operand V^T follows, read from a
// key-pair-transposed V tile in LDS.  The backward uses the same device:
// every product is arranged so that the operand built from a score-shaped
// tile is the one whose contraction runs over that tile's rows.
//
// Head dimension 128; sequence length any (the last key and query blocks
// are masked); full or causal.  The log-sum-exp of every query row (natural
// log) is stored for the backward.
#include "fp4q_launch.hpp"
#include "lane_ops.hpp"

#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>
#include <utility>

namespace fp4q {

namespace {

// Static scratch of the allocation-free backward (fp4q_attn_bwd_noalloc):
// D of up to kAttnScratchRows query rows.  Each GPU holds its own copy for
// the life of the process; host code reaches it only through the address
// hipGetSymbolAddress returns on that device (attn_noalloc_scratch).
__device__ __align__(256) float scratch[kAttnScratchRows];

typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;             // head dimension
constexpr int kThreads = 256;       // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename F, int... I>
__device__ __forceinline__ void sfor_impl(F&& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>()), ...);
}
template <int N, typename F>
__device__ __forceinline__ void sfor(F&& f)
{
    sfor_impl(f, std::make_integer_sequence<int, N>());
}

// Element `col` of row `row` of a head's slice: the head's base is uniform
// (scalar registers) and the rest a 32-bit offset, which the loads take as a
// vector offset on a scalar base (the host keeps every head's slice of
// every tensor below 2 GiB).
template <typename T>
__device__ __forceinline__ const T* head_at(const T* base, int64_t head_row, int64_t ld, int row, int col)
{
    return base + head_row * ld + (uint32_t)(row * (uint32_t)ld + col);
}

// A buffer resource over rows [r0, L) of one head's slice of a row-major
// tensor (ld elements per row): a load at a row past the sequence lies past
// the resource and reads as zero, so the next-block loads need no masks, and
// their per-lane offsets do not change from block to block.  Needs
// r0 < L; the extent fits 32 bits because a head's slice of every operand is
// below 2^31 elements (checked at the entry points).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const T* base, int64_t head_row, int64_t ld, int r0, int L)
{
    const uint32_t bytes = (uint32_t)(L - r0) * (uint32_t)ld * (uint32_t)sizeof(T);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(head_at(base, head_row, ld, r0, 0)), (short)0, (int)bytes,
                                             0x00020000);
}

// 2^(b - 127) as a float (b = 0: the subnormal 2^-127).
__device__ __forceinline__ float e8m0_f32(uint32_t b)
{
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// 8 E4M3 bytes times one E8M0 scale -> 8 bf16 (exact).
__device__ __forceinline__ v8bf cvt8_e4m3(v2u raw, float scale)
{
    const bf16x2 a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, false);
    const bf16x2 a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.x, scale, true);
    const bf16x2 a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, false);
    const bf16x2 a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw.y, scale, true);
    return __builtin_bit_cast(v8bf, (v4u){__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1),
                                          __builtin_bit_cast(uint32_t, a2), __builtin_bit_cast(uint32_t, a3)});
}

// Two floats -> one dword of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ v16f mfma_bf16(v8bf a, v8bf b, v16f c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16f zero16()
{
    v16f z;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        z[r] = 0.0f;
    return z;
}

// Pair-transposed tiles.  A [64 x 128] bf16 tile X (rows: keys or queries)
// is stored transposed with row pairs packed: row d of the stored tile holds
// the dwords (X[2p][d], X[2p+1][d]).  Within each group of 16 rows (8 pairs)
// the pairs are ordered so that the 8 rows one MFMA lane half contracts over
// in a 16-row step -- rows 4h .. 4h+3 and 8+4h .. 8+4h+3 of the group, the
// order in which a score tile's registers hold them -- are 16 contiguous
// bytes: pair q of a group goes to dword slot q with bits 1 and 2 swapped.
// One 16-byte read per operand then, and at a 144-byte row pitch the 16
// lanes of a read cycle hit distinct banks.
__device__ __forceinline__ int pair_slot(int p)
{
    return (p & ~7) | (p & 1) | ((p & 2) << 1) | ((p & 4) >> 1);
}

// `lo`, `hi`: 8 bf16 (d-chunk `dchunk` of 8) of rows 2p and 2p+1.
__device__ __forceinline__ void store_pair_t(uint8_t* tt, int pitch, int dchunk, int p, v4u lo, v4u hi)
{
    uint8_t* base = tt + (8 * dchunk) * pitch + 4 * pair_slot(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint32_t*>(base + (2 * e) * pitch) = (lo[e] & 0xFFFFu) | (hi[e] << 16);
        *reinterpret_cast<uint32_t*>(base + (2 * e + 1) * pitch) = (lo[e] >> 16) | (hi[e] & 0xFFFF0000u);
    }
}

// The 8-value A operand of a product whose contraction runs over the rows of
// a pair-transposed tile: stored row `row`, the 16-row step covering tile
// rows [32 sb + 16 tp, +16), this lane half's 8 of them.
__device__ __forceinline__ v8bf read_pair_t(const uint8_t* tt, int pitch, int row, int sb, int tp, int h)
{
    return *reinterpret_cast<const v8bf*>(tt + row * pitch + 2 * (32 * sb + 16 * tp) + 16 * h);
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
constexpr int kFwdQ = 128;                  // queries per workgroup (32 per wave)
constexpr int kFwdK = 64;                   // keys per step
constexpr int kKbPitch = 272;               // bytes per key row of the bf16 K tile (68 dwords: conflict-free)
constexpr int kVtPitch = 144;               // bytes per d row of the key-pair-transposed V tile
constexpr int kFwdKBytes = kFwdK * kKbPitch;          // 17408
constexpr int kFwdVBytes = kD * kVtPitch;             // 18432
constexpr int kFwdBuf = kFwdKBytes + kFwdVBytes;      // 35840; two buffers, two workgroups per CU

// Registers holding one key block on its way from memory to LDS.
struct FwdStage {
    v4u k[2];         // 16 E4M3 codes of one key
    uint32_t ks[2];   // that key's scale dword (4 E8M0 bytes)
    v4u v[2][2];
};

// Per-lane byte offsets of the next-block loads inside a block (the same
// for every block).
struct FwdOff {
    uint32_t k[2], ks[2], v[2][2];
};

__device__ __forceinline__ FwdOff fwd_offsets(const AttnArgs& a)
{
    const int t = threadIdx.x;
    FwdOff o;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = t + kThreads * i, key = u >> 3, c = u & 7;
        o.k[i] = (uint32_t)(key * a.ldk + 16 * c);
        o.ks[i] = (uint32_t)(key * a.ldks);
        const int p = u & 31, dc = u >> 5;
#pragma unroll
        for (int e = 0; e < 2; ++e)
            o.v[i][e] = (uint32_t)(((2 * p + e) * a.ldv + 8 * dc) * 2);
    }
    return o;
}

__device__ __forceinline__ void fwd_load(FwdStage& st, const AttnArgs& a, const FwdOff& o, int64_t head_row, int k0)
{
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(a.kc, head_row, a.ldk, k0, a.L);
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(a.ks, head_row, a.ldks, k0, a.L);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(a.v, head_row, a.ldv, k0, a.L);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        st.k[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)o.k[i], 0, 0);
        st.ks[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)o.ks[i], 0, 0);
#pragma unroll
        for (int e = 0; e < 2; ++e)
            st.v[i][e] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)o.v[i][e], 0, 0);
    }
}

// K is converted to bf16 here, once per block for the whole workgroup (each
// code times its group's E8M0 scale, exact), so the waves read MFMA operands
// straight from LDS.
__device__ __forceinline__ void fwd_store(const FwdStage& st, uint8_t* buf)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = t + kThreads * i, key = u >> 3, c = u & 7;
        const float sc = e8m0_f32((st.ks[i] >> (8 * (c >> 1))) & 0xFFu);
        uint8_t* kr = buf + key * kKbPitch + 32 * c;
        *reinterpret_cast<v8bf*>(kr) = cvt8_e4m3((v2u){st.k[i].x, st.k[i].y}, sc);
        *reinterpret_cast<v8bf*>(kr + 16) = cvt8_e4m3((v2u){st.k[i].z, st.k[i].w}, sc);
        // V^T, key pairs packed (keys 2p, 2p+1 of d-chunk dc)
        const int p = u & 31, dc = u >> 5;
        store_pair_t(buf + kFwdKBytes, kVtPitch, dc, p, st.v[i][0], st.v[i][1]);
    }
}

template <bool CAUSAL, bool OBF>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    // blockIdx.x: head, blockIdx.y: query block, the last (longest causal
    // rows) first -- the dispatcher walks x fastest, so every head's long
    // blocks start before any short one
    const int nqb = (a.L + kFwdQ - 1) / kFwdQ;
    const int qb = nqb - 1 - (int)blockIdx.y;
    const int64_t head_row = (int64_t)blockIdx.x * a.L;
    const int q0 = qb * kFwdQ + 32 * wave;      // the wave's first query
    const int q = q0 + l32;                     // this lane's query

    // Q of this lane's query as the B operand of S^T = K Q^T: 8 steps of d.
    v8bf qb16[8];
    {
        const bool ok = q < a.L;
        const uint32_t sc = ok ? *reinterpret_cast<const uint32_t*>(a.qs + (head_row + q) * a.ldqs) : 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const v2u raw = ok ? *reinterpret_cast<const v2u*>(a.qc + (head_row + q) * a.ldq + 16 * t + 8 * h)
                               : (v2u){0u, 0u};
            qb16[t] = cvt8_e4m3(raw, e8m0_f32((sc >> (8 * (t >> 1))) & 0xFFu));
        }
    }
    v16f o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = zero16();
    float m = -INFINITY, l = 0.0f;
    const float c = a.scale * kLog2e;           // scores in log2 units

    const int nkb_all = (a.L + kFwdK - 1) / kFwdK;
    const int nkb = CAUSAL ? min(nkb_all, (qb * kFwdQ + kFwdQ - 1) / kFwdK + 1) : nkb_all;
    FwdStage st;
    const FwdOff fo = fwd_offsets(a);
    fwd_load(st, a, fo, head_row, 0);
    fwd_store(st, lds);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const uint8_t* buf = lds + (kb & 1) * kFwdBuf;
        const int k0 = kb * kFwdK;
        if (kb + 1 < nkb)
            fwd_load(st, a, fo, head_row, k0 + kFwdK);

    // S^T for the 64 keys: two 32-key sub-blocks.
        v16f s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const uint8_t* kr = buf + (32 * sb + l32) * kKbPitch + 16 * h;
            s[sb] = zero16();
#pragma unroll
            for (int t = 0; t < 8; ++t)
                s[sb] = mfma_bf16(*reinterpret_cast<const v8bf*>(kr + 32 * t), qb16[t], s[sb]);
        }
        // mask keys past the sequence and (causal) after the query
        const bool edge = k0 + kFwdK > a.L || (CAUSAL && k0 + kFwdK - 1 > q0);
        if (edge) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (key >= a.L || (CAUSAL && key > q))
                        s[sb][r] = -INFINITY;
                }
        }
        // online softmax of this lane's query
        float mx = -INFINITY;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                mx = fmaxf(mx, s[sb][r]);
        mx = fmax_xor32(mx);
        // Lazy rescaling: the reference m moves only when this block's max
        // passes it by more than 8 in log2 units (or m is still -inf; both
        // -inf gives NaN, no move), so P = exp2(c s - c m) stays below 2^8,
        // and O and l are rescaled only when some row of the wave moved.
        const bool grow = c * (mx - m) > 8.0f;
        const float m_new = grow ? mx : m;
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        const float cm = c * m_use;
        float rs = 0.0f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[sb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(c, s[sb][r], -cm));
                rs += s[sb][r];
            }
        rs = fadd_xor32(rs);
        if (__any(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(c * (m - m_use)) : 1.0f;
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    o[i][r] *= alpha;
        }
        l += rs;
        m = m_new;
        // O^T += V^T P^T over four 16-key steps
        const uint8_t* vt = buf + kFwdKBytes;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int sb = t4 >> 1, tp = t4 & 1;
            const v4u pw = {pack_bf16(s[sb][8 * tp + 0], s[sb][8 * tp + 1]), pack_bf16(s[sb][8 * tp + 2], s[sb][8 * tp + 3]),
                            pack_bf16(s[sb][8 * tp + 4], s[sb][8 * tp + 5]), pack_bf16(s[sb][8 * tp + 6], s[sb][8 * tp + 7])};
            const v8bf pb = __builtin_bit_cast(v8bf, pw);
#pragma unroll
            for (int db = 0; db < 4; ++db)
                o[db] = mfma_bf16(read_pair_t(vt, kVtPitch, 32 * db + l32, sb, tp, h), pb, o[db]);
        }
        if (kb + 1 < nkb) {
            // every wave left the other buffer at the previous step's barrier
            fwd_store(st, lds + ((kb + 1) & 1) * kFwdBuf);
            __syncthreads();
        }
    }
    // O = O^T / l; lse = ln(l) + scale * m
    if (q < a.L) {
        const float inv = 1.0f / l;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * db + 8 * g4 + 4 * h;
                const float x0 = o[db][4 * g4] * inv, x1 = o[db][4 * g4 + 1] * inv;
                const float x2 = o[db][4 * g4 + 2] * inv, x3 = o[db][4 * g4 + 3] * inv;
                if (OBF) {
                    v2u w = {pack_bf16(x0, x1), pack_bf16(x2, x3)};
                    *reinterpret_cast<v2u*>(reinterpret_cast<__bf16*>(a.o) + (head_row + q) * a.ldo + d) = w;
                } else {
                    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.o) + (head_row + q) * a.ldo + d) =
                        make_float4(x0, x1, x2, x3);
                }
            }
        if (h == 0)
            a.lse[head_row + q] = (__builtin_amdgcn_logf(l) + c * m) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Backward.  D_i = sum_d dO_id O_id first (one thread per row), then
//   dQ kernel   (128 queries per workgroup, over key blocks of 64):
//     S^T = K Q^T, P^T = exp2(c S^T - lse2), dP^T = V dO^T,
//     dS^T = P^T (dP^T - D), dQ^T += K^T dS^T;
//   dK/dV kernel (128 keys per workgroup, over query blocks of 64):
//     S = Q K^T, P = exp2(c S - lse2), dP = dO V^T, dS = P (dP - D),
//     dV += P^T dO, dK += dS^T Q.
// Both recompute the scores, so no partial sums cross workgroups.
// ---------------------------------------------------------------------------
template <bool OBF>
__global__ __launch_bounds__(kThreads) void attn_delta_kernel(AttnArgs a)
{
    const int64_t row = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (row >= (int64_t)a.bh * a.L)
        return;
    const uint16_t* g = a.dout + row * a.lddo;
    float acc = 0.0f;
#pragma unroll 4
    for (int c = 0; c < kD / 8; ++c) {
        const v4u gw = *reinterpret_cast<const v4u*>(g + 8 * c);
        float ov[8];
        if (OBF) {
            const v4u ow = *reinterpret_cast<const v4u*>(reinterpret_cast<const uint16_t*>(a.o) + row * a.ldo + 8 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ov[2 * e] = __uint_as_float(ow[e] << 16);
                ov[2 * e + 1] = __uint_as_float(ow[e] & 0xFFFF0000u);
            }
        } else {
            const float* op = reinterpret_cast<const float*>(a.o) + row * a.ldo + 8 * c;
            const float4 x0 = *reinterpret_cast<const float4*>(op), x1 = *reinterpret_cast<const float4*>(op + 4);
            ov[0] = x0.x; ov[1] = x0.y; ov[2] = x0.z; ov[3] = x0.w;
            ov[4] = x1.x; ov[5] = x1.y; ov[6] = x1.z; ov[7] = x1.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = __builtin_fmaf(__uint_as_float(gw[e] << 16), ov[2 * e], acc);
            acc = __builtin_fmaf(__uint_as_float(gw[e] & 0xFFFF0000u), ov[2 * e + 1], acc);
        }
    }
    a.delta[row] = acc;
}

// Registers of a score-shaped tile (16 of them, rows 8(r/4) + 4h + r%4),
// its 16-row step tp as the 8-value operand of the next product, in bf16.
__device__ __forceinline__ v8bf pack_step(const v16f& x, int tp)
{
    const v4u w = {pack_bf16(x[8 * tp + 0], x[8 * tp + 1]), pack_bf16(x[8 * tp + 2], x[8 * tp + 3]),
                   pack_bf16(x[8 * tp + 4], x[8 * tp + 5]), pack_bf16(x[8 * tp + 6], x[8 * tp + 7])};
    return __builtin_bit_cast(v8bf, w);
}

// ---- dQ ----
constexpr int kDqQ = 128;                  // queries per workgroup
constexpr int kDqK = 64;                   // keys per step
constexpr int kRowPitch = 272;             // bytes per row of a row-major bf16 [64 x 128] tile
constexpr int kDqKb = kDqK * kRowPitch;    // K row-major bf16 (converted once per block)
constexpr int kDqV = kDqK * kRowPitch;     // V row-major bf16
constexpr int kDqKt = kD * kVtPitch;       // K^T bf16 (key pairs)
constexpr int kDqBuf = kDqKb + kDqV + kDqKt;

struct DqStage {
    v2u kc[2][2];   // K codes of keys 2p, 2p+1, 8 bytes at d-chunk dc
    uint32_t ksb[2][2];
    v4u v[2][2];    // V rows 2p, 2p+1, d-chunk dc (8 bf16)
};

// Per-lane byte offsets of the next-block loads inside a block, for keys
// 2p + e; the second half of the threads' columns (i = 1) lies 64 bytes
// (codes), 2 bytes (scales) and 128 bytes (V) further on.
struct DqOff {
    uint32_t kc[2], ks[2], v[2];
};

__device__ __forceinline__ DqOff dq_offsets(const AttnArgs& a)
{
    const int t = threadIdx.x, p = t & 31, dc = t >> 5;
    DqOff o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int key = 2 * p + e;
        o.kc[e] = (uint32_t)(key * a.ldk + 8 * dc);
        o.ks[e] = (uint32_t)(key * a.ldks + (dc >> 2));
        o.v[e] = (uint32_t)((key * a.ldv + 8 * dc) * 2);
    }
    return o;
}

__device__ __forceinline__ void dq_load(DqStage& st, const AttnArgs& a, const DqOff& o, int64_t head_row, int k0)
{
    const __amdgpu_buffer_rsrc_t rk = rows_rsrc(a.kc, head_row, a.ldk, k0, a.L);
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(a.ks, head_row, a.ldks, k0, a.L);
    const __amdgpu_buffer_rsrc_t rv = rows_rsrc(a.v, head_row, a.ldv, k0, a.L);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            st.kc[i][e] = __builtin_amdgcn_raw_buffer_load_b64(rk, (int)(o.kc[e] + 64 * i), 0, 0);
            st.ksb[i][e] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)(o.ks[e] + 2 * i), 0, 0);
            st.v[i][e] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(o.v[e] + 128 * i), 0, 0);
        }
}

__device__ __forceinline__ void dq_store(const DqStage& st, uint8_t* buf)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = t + kThreads * i, p = u & 31, dc = u >> 5;
        v4u kb[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int key = 2 * p + e;
            kb[e] = __builtin_bit_cast(v4u, cvt8_e4m3(st.kc[i][e], e8m0_f32(st.ksb[i][e])));
            *reinterpret_cast<v4u*>(buf + key * kRowPitch + 16 * dc) = kb[e];
            *reinterpret_cast<v4u*>(buf + kDqKb + key * kRowPitch + 16 * dc) = st.v[i][e];
        }
        store_pair_t(buf + kDqKb + kDqV, kVtPitch, dc, p, kb[0], kb[1]);
    }
}

template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_dq_kernel(AttnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int nqb = (a.L + kDqQ - 1) / kDqQ;
    const int qb = nqb - 1 - (int)blockIdx.y;   // as in the forward: long blocks first
    const int64_t head_row = (int64_t)blockIdx.x * a.L;
    const int q0 = qb * kDqQ + 32 * wave;
    const int q = q0 + l32;
    const bool qok = q < a.L;
    const float c = a.scale * kLog2e;

    // this lane's query: Q (B operand of S^T = K Q^T), dO (B operand of
    // dP^T = V dO^T), lse in log2 units, D
    v8bf qb16[8], gb16[8];
    {
        const uint32_t sc = qok ? *reinterpret_cast<const uint32_t*>(a.qs + (head_row + q) * a.ldqs) : 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const v2u raw = qok ? *reinterpret_cast<const v2u*>(a.qc + (head_row + q) * a.ldq + 16 * t + 8 * h)
                                : (v2u){0u, 0u};
            qb16[t] = cvt8_e4m3(raw, e8m0_f32((sc >> (8 * (t >> 1))) & 0xFFu));
            const v4u gw = qok ? *reinterpret_cast<const v4u*>(a.dout + (head_row + q) * a.lddo + 16 * t + 8 * h)
                               : (v4u){0u, 0u, 0u, 0u};
            gb16[t] = __builtin_bit_cast(v8bf, gw);
        }
    }
    const float lse2 = qok ? a.lse[head_row + q] * kLog2e : 0.0f;
    const float dlt = qok ? a.delta[head_row + q] : 0.0f;
    v16f dq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        dq[i] = zero16();

    // One LDS buffer: the next key block is loaded into registers during a
    // step and stored between the step's two barriers.  Two workgroups per
    // CU (two waves per SIMD) hide each other's latencies.
    const int nkb_all = (a.L + kDqK - 1) / kDqK;
    const int nkb = CAUSAL ? min(nkb_all, (qb * kDqQ + kDqQ - 1) / kDqK + 1) : nkb_all;
    const uint8_t* buf = lds;
    const uint8_t* kt = buf + kDqKb + kDqV;
    DqStage st;
    const DqOff qo = dq_offsets(a);
    dq_load(st, a, qo, head_row, 0);
    dq_store(st, lds);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int k0 = kb * kDqK;
        if (kb + 1 < nkb)
            dq_load(st, a, qo, head_row, k0 + kDqK);
        const bool edge = k0 + kDqK > a.L || (CAUSAL && k0 + kDqK - 1 > q0);
        // one 32-key half at a time: S^T, dP^T, dS^T = P^T (dP^T - D) with
        // P^T = 0 for keys past the sequence, (causal) after the query, and
        // for queries past the sequence; then dQ^T += K^T dS^T
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int key = 32 * sb + l32;
            v16f sv = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const v8bf kw = *reinterpret_cast<const v8bf*>(buf + key * kRowPitch + 32 * t + 16 * h);
                sv = mfma_bf16(kw, qb16[t], sv);
                const v8bf vw = *reinterpret_cast<const v8bf*>(buf + kDqKb + key * kRowPitch + 32 * t + 16 * h);
                dp = mfma_bf16(vw, gb16[t], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(c, sv[r], -lse2));
                if (edge) {
                    const int kk = k0 + 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (kk >= a.L || (CAUSAL && kk > q))
                        pv = 0.0f;
                }
                sv[r] = qok ? pv * (dp[r] - dlt) : 0.0f;
            }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                const v8bf bds = pack_step(sv, tp);
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    dq[db] = mfma_bf16(read_pair_t(kt, kVtPitch, 32 * db + l32, sb, tp, h), bds, dq[db]);
            }
        }
        if (kb + 1 < nkb) {
            __syncthreads();   // every wave is done with the buffer
            dq_store(st, lds);
            __syncthreads();
        }
    }
    if (qok) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = 32 * db + 8 * g4 + 4 * h;
                *reinterpret_cast<float4*>(a.dq + (head_row + q) * a.ldg + d) =
                    make_float4(a.scale * dq[db][4 * g4], a.scale * dq[db][4 * g4 + 1], a.scale * dq[db][4 * g4 + 2],
                                a.scale * dq[db][4 * g4 + 3]);
            }
    }
}

// ---- dK, dV ----
constexpr int kDkK = 128;                  // keys per workgroup
constexpr int kDkQ = 64;                   // queries per step
constexpr int kDkQb = kDkQ * kRowPitch;    // Q row-major bf16 (converted once per block)
constexpr int kDkQt = kD * kVtPitch;       // Q^T bf16 (query pairs)
constexpr int kDkG = kDkQ * kRowPitch;     // dO row-major
constexpr int kDkGt = kD * kVtPitch;       // dO^T (query pairs)
constexpr int kDkL = kDkQ * 4;             // lse (log2 units) of the queries
constexpr int kDkDl = kDkQ * 4;            // D of the queries
constexpr int kDkBuf = kDkQb + kDkQt + kDkG + kDkGt + kDkL + kDkDl;

// Raw loaded words only: arithmetic on a loaded value here would make the
// compiler wait for that load (and, loads completing in order, for every
// load before it) at once, instead of at the LDS store a step later.
struct DkStage {
    v2u qc[2][2];
    uint32_t qs[2];   // the scale dwords (4 E8M0 bytes) of query rows 2p and 2p+1
    v4u g[2][2];
    float ls, dl;     // lse (natural log) and D of query t
};

// Per-lane byte offsets of the next-block loads inside a block, for queries
// 2p + e; the second half of the threads' columns (i = 1) lies 64 bytes
// (codes) and 128 bytes (dO) further on.
struct DkOff {
    uint32_t qc[2], qs[2], g[2];
};

__device__ __forceinline__ DkOff dk_offsets(const AttnArgs& a)
{
    const int t = threadIdx.x, p = t & 31, dc = t >> 5;
    DkOff o;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int q = 2 * p + e;
        o.qc[e] = (uint32_t)(q * a.ldq + 8 * dc);
        o.qs[e] = (uint32_t)(q * a.ldqs);
        o.g[e] = (uint32_t)((q * a.lddo + 8 * dc) * 2);
    }
    return o;
}

__device__ __forceinline__ void dk_load(DkStage& st, const AttnArgs& a, const DkOff& o, int64_t head_row, int i0)
{
    const int t = threadIdx.x;
    const __amdgpu_buffer_rsrc_t rq = rows_rsrc(a.qc, head_row, a.ldq, i0, a.L);
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(a.qs, head_row, a.ldqs, i0, a.L);
    const __amdgpu_buffer_rsrc_t rg = rows_rsrc(a.dout, head_row, a.lddo, i0, a.L);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            st.qc[i][e] = __builtin_amdgcn_raw_buffer_load_b64(rq, (int)(o.qc[e] + 64 * i), 0, 0);
            if (i == 0)   // the same rows for i = 1
                st.qs[e] = __builtin_amdgcn_raw_buffer_load_b32(rs, (int)o.qs[e], 0, 0);
            st.g[i][e] = __builtin_amdgcn_raw_buffer_load_b128(rg, (int)(o.g[e] + 128 * i), 0, 0);
        }
    const __amdgpu_buffer_rsrc_t rl = rows_rsrc(a.lse, head_row, 1, i0, a.L);
    const __amdgpu_buffer_rsrc_t rd = rows_rsrc(a.delta, head_row, 1, i0, a.L);
    st.ls = __uint_as_float(t < kDkQ ? __builtin_amdgcn_raw_buffer_load_b32(rl, 4 * t, 0, 0) : 0u);
    st.dl = __uint_as_float(t < kDkQ ? __builtin_amdgcn_raw_buffer_load_b32(rd, 4 * t, 0, 0) : 0u);
}

// The dV kernel reads Q (rows) and dO^T (pairs); the dK kernel Q (rows),
// Q^T (pairs), dO (rows) and D.  Each stores only its own tiles.
template <bool DV>
__device__ __forceinline__ void dk_store(const DkStage& st, uint8_t* buf)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int u = t + kThreads * i, p = u & 31, dc = u >> 5;
        v4u qb[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int qq = 2 * p + e;
            qb[e] = __builtin_bit_cast(v4u, cvt8_e4m3(st.qc[i][e], e8m0_f32((st.qs[e] >> (8 * (dc >> 2))) & 0xFFu)));
            *reinterpret_cast<v4u*>(buf + qq * kRowPitch + 16 * dc) = qb[e];
            if constexpr (!DV)
                *reinterpret_cast<v4u*>(buf + kDkQb + kDkQt + qq * kRowPitch + 16 * dc) = st.g[i][e];
        }
        if constexpr (DV)
            store_pair_t(buf + kDkQb + kDkQt + kDkG, kVtPitch, dc, p, st.g[i][0], st.g[i][1]);
        else
            store_pair_t(buf + kDkQb, kVtPitch, dc, p, qb[0], qb[1]);
    }
    if (t < kDkQ) {
        reinterpret_cast<float*>(buf + kDkQb + kDkQt + kDkG + kDkGt)[t] = st.ls * kLog2e;
        if constexpr (!DV)
            reinterpret_cast<float*>(buf + kDkQb + kDkQt + kDkG + kDkGt + kDkL)[t] = st.dl;
    }
}

// DV: dV += P^T dO (needs S only); else dK += dS^T Q (needs S and dP).  Two
// kernels rather than one, so each fits two waves per SIMD; both recompute S.
template <bool CAUSAL, bool DV>
__global__ __launch_bounds__(kThreads, 2) void attn_dkdv_kernel(AttnArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, h = lane >> 5;
    const int kb = (int)blockIdx.y;             // causal: the first key blocks see the most queries
    const int64_t head_row = (int64_t)blockIdx.x * a.L;
    const int j0 = kb * kDkK + 32 * wave;       // the wave's first key
    const int j = j0 + l32;                     // this lane's key
    const bool kok = j < a.L;
    const float c = a.scale * kLog2e;

    // this lane's key: K (B operand of S = Q K^T), V (B operand of dP = dO V^T)
    v8bf kb16[8], vb16[DV ? 1 : 8];
    {
        const uint32_t sc = kok ? *reinterpret_cast<const uint32_t*>(a.ks + (head_row + j) * a.ldks) : 0u;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const v2u raw = kok ? *reinterpret_cast<const v2u*>(a.kc + (head_row + j) * a.ldk + 16 * t + 8 * h)
                                : (v2u){0u, 0u};
            kb16[t] = cvt8_e4m3(raw, e8m0_f32((sc >> (8 * (t >> 1))) & 0xFFu));
            if constexpr (!DV) {
                const v4u vw = kok ? *reinterpret_cast<const v4u*>(a.v + (head_row + j) * a.ldv + 16 * t + 8 * h)
                                   : (v4u){0u, 0u, 0u, 0u};
                vb16[t] = __builtin_bit_cast(v8bf, vw);
            }
        }
    }
    v16f acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc[i] = zero16();
    // One LDS buffer (see the dQ kernel), two workgroups per CU.
    const int nib = (a.L + kDkQ - 1) / kDkQ;
    const int ib0 = CAUSAL ? (kb * kDkK) / kDkQ : 0;   // the first query block that sees a key of the tile
    const uint8_t* buf = lds;
    const uint8_t* qt = buf + kDkQb;
    const uint8_t* g = qt + kDkQt;
    const uint8_t* gt = g + kDkG;
    const float* lsv = reinterpret_cast<const float*>(gt + kDkGt);
    const float* dlv = lsv + kDkQ;
    DkStage st;
    const DkOff ko = dk_offsets(a);
    dk_load(st, a, ko, head_row, ib0 * kDkQ);
    dk_store<DV>(st, lds);
    __syncthreads();
    for (int ib = ib0; ib < nib; ++ib) {
        const int i0 = ib * kDkQ;
        if (DV && ib + 1 < nib)
            dk_load(st, a, ko, head_row, i0 + kDkQ);
        // rows = queries 32 qs + 8(r/4) + 4h + r%4; zero past the sequence
        // and (causal) where the key follows the query
        const bool edge = i0 + kDkQ > a.L || (CAUSAL && i0 < j0 + 31);
        // one 32-query half at a time: S = Q K^T, P = exp2(c S - lse2),
        // then dV += P^T dO, or dP = dO V^T, dS = P (dP - D), dK += dS^T Q,
        // over the half's two 16-query steps
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            // the dK kernel's loads of the next query block go out with the
            // second half, so their registers are live for half a step (the
            // dV kernel has the registers to issue them at the top)
            if (!DV && qs == 1 && ib + 1 < nib)
                dk_load(st, a, ko, head_row, i0 + kDkQ);
            const int qr0 = 32 * qs + l32;
            v16f sv = zero16(), dp = zero16();
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const v8bf qw = *reinterpret_cast<const v8bf*>(buf + qr0 * kRowPitch + 32 * t + 16 * h);
                sv = mfma_bf16(qw, kb16[t], sv);
                if constexpr (!DV) {
                    const v8bf gw = *reinterpret_cast<const v8bf*>(g + qr0 * kRowPitch + 32 * t + 16 * h);
                    dp = mfma_bf16(gw, vb16[t], dp);
                }
            }
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int qr = 32 * qs + 8 * g4 + 4 * h;
                const float4 l4 = *reinterpret_cast<const float4*>(lsv + qr);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                float dv4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if constexpr (!DV) {
                    const float4 d4 = *reinterpret_cast<const float4*>(dlv + qr);
                    dv4[0] = d4.x; dv4[1] = d4.y; dv4[2] = d4.z; dv4[3] = d4.w;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g4 + e;
                    float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(c, sv[r], -lv[e]));
                    if (edge) {
                        const int qq = i0 + qr + e;
                        if (qq >= a.L || (CAUSAL && j > qq))
                            pv = 0.0f;
                    }
                    if constexpr (DV)
                        sv[r] = pv;
                    else
                        sv[r] = pv * (dp[r] - dv4[e]);
                }
            }
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                const v8bf ob = pack_step(sv, tp);
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    acc[db] = mfma_bf16(ob, read_pair_t(DV ? gt : qt, kVtPitch, 32 * db + l32, qs, tp, h), acc[db]);
            }
        }
        if (ib + 1 < nib) {
            __syncthreads();   // every wave is done with the buffer
            dk_store<DV>(st, lds);
            __syncthreads();
        }
    }
    // dV[key][d] or dK[key][d]: lane holds column d = 32 db + l32, keys
    // j0 + 8(r/4) + 4h + r%4
    float* out = DV ? a.dv : a.dk;
    const float mul = DV ? 1.0f : a.scale;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = j0 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (key < a.L)
                out[(head_row + key) * a.ldg + 32 * db + l32] = mul * acc[db][r];
        }
}

} // namespace

hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t s)
{
    const int64_t rows = (int64_t)a.bh * a.L;
    hipLaunchKernelGGL((a.o_bf16 ? attn_delta_kernel<true> : attn_delta_kernel<false>),
                       dim3((unsigned)((rows + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    constexpr size_t kDqLds = kDqBuf, kDkLds = kDkBuf;
    static_assert(2 * kDqLds <= 160 * 1024 && 2 * kDkLds <= 160 * 1024, "two workgroups per CU");
    auto raise = [](const void* fn, size_t bytes) {
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    };
    const void* dqf = a.causal ? reinterpret_cast<const void*>(attn_dq_kernel<true>)
                               : reinterpret_cast<const void*>(attn_dq_kernel<false>);
    const void* dvf = a.causal ? reinterpret_cast<const void*>(attn_dkdv_kernel<true, true>)
                               : reinterpret_cast<const void*>(attn_dkdv_kernel<false, true>);
    const void* dkf = a.causal ? reinterpret_cast<const void*>(attn_dkdv_kernel<true, false>)
                               : reinterpret_cast<const void*>(attn_dkdv_kernel<false, false>);
    if ((e = raise(dqf, kDqLds)) != hipSuccess || (e = raise(dvf, kDkLds)) != hipSuccess ||
        (e = raise(dkf, kDkLds)) != hipSuccess)
        return e;
    const dim3 gq(a.bh, (a.L + kDqQ - 1) / kDqQ), gk(a.bh, (a.L + kDkK - 1) / kDkK);
    if (a.causal) {
        hipLaunchKernelGGL(attn_dq_kernel<true>, gq, dim3(kThreads), kDqLds, s, a);
        hipLaunchKernelGGL((attn_dkdv_kernel<true, true>), gk, dim3(kThreads), kDkLds, s, a);
        hipLaunchKernelGGL((attn_dkdv_kernel<true, false>), gk, dim3(kThreads), kDkLds, s, a);
    } else {
        hipLaunchKernelGGL(attn_dq_kernel<false>, gq, dim3(kThreads), kDqLds, s, a);
        hipLaunchKernelGGL((attn_dkdv_kernel<false, true>), gk, dim3(kThreads), kDkLds, s, a);
        hipLaunchKernelGGL((attn_dkdv_kernel<false, false>), gk, dim3(kThreads), kDkLds, s, a);
    }
    return hipGetLastError();
}

hipError_t attn_noalloc_scratch(float** p)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // once per device, with that device current: the device address of
        // this GPU's copy of the array
        void* q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = static_cast<float*>(q);
    }
    *p = addr[dev];
    return hipSuccess;
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s)
{
    constexpr size_t kFwdLds = 2 * kFwdBuf;
    static_assert(2 * kFwdLds <= 160 * 1024, "two forward workgroups per CU");
    const dim3 grid(a.bh, (a.L + kFwdQ - 1) / kFwdQ);
    auto fn = a.causal ? (a.o_bf16 ? attn_fwd_kernel<true, true> : attn_fwd_kernel<true, false>)
                       : (a.o_bf16 ? attn_fwd_kernel<false, true> : attn_fwd_kernel<false, false>);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kFwdLds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(fn, grid, dim3(kThreads), kFwdLds, s, a);
    return hipGetLastError();
}

} // namespace fp4q
