// Split-K paged decode attention over a list of pages, and the log-sum-exp merge.
//
// EntmaxKV README, introduction: attention is exact over the selected pages; LOCKS
// README, "How it works": the paged attention kernel reads only the selected pages.
// The same kernel, walking every page of the block table, is the dense baseline.
//
// Work decomposition: one workgroup per (sequence s, KV head g, split); a split is up to
// `pps` consecutive entries of the unit's page list. Each wave owns a tile of 16 query
// heads of the group (G <= 16: one wave, heads past G are zero padding; G = 128: eight
// waves). Per 16-token page a wave computes
//   S^T[token, head] = K_page[16 x D] . Q_tile^T         (MFMA 16x16x32 bf16, fp32 acc)
// so that each lane holds one head's scores for 4 tokens, runs the online softmax in
// fp32 (base-2 exponent with scale*log2(e) folded in), and accumulates
//   O[head, d] += P[head, token] . V_page[token, d]     (MFMA 16x16x16 bf16, fp32 acc)
// with P split into bf16 hi + lo parts, so P keeps ~16 mantissa bits. V's columns are
// assigned to MFMA columns as d = lane_col * (Dv / 16) + c so that each lane loads
// contiguous bytes of V rows and a 16-byte load serves 8 MFMAs. fp32 caches are fed to
// the same MFMAs as bf16 hi + lo pairs (three products: hi*hi + lo*hi + hi*lo).
// Slots past the sequence length (tail page only) are masked in S and zeroed in V.
// A wave writes unnormalised fp32 partials (m, l, acc) per head; lse_merge_kernel
// combines the splits: M = max m_i, out = sum acc_i 2^(m_i - M) / sum l_i 2^(m_i - M).
#include "attn_core.h"

namespace psd {
namespace {

// ---- latent (MLA-style) attention: K and V rows are one 576-dim latent row -------------
//
// For many-head groups (G = 16 * WAVES, up to 128) on a latent cache (V = first 512 dims of
// each K row, same pointer and strides), a workgroup stages each 16-token page once in
// LDS (direct-to-LDS loads, rows padded to 73 16-byte pieces so that fragment reads are
// conflict-free), three pages deep, and every wave reads its MFMA fragments from there;
// each wave keeps its 16 heads' q in registers. V columns map to MFMA columns as
// d = 128 w + 8 lane_col + cc for tile 8 w + cc, so that a lane's 16-byte read serves
// 8 tiles and the 16 lanes of a row read 16 consecutive pieces.
constexpr int kLatRowPieces = 73;                 // 72 pieces of 16 B + 1 pad
constexpr int kLatLoads = (16 * kLatRowPieces + 63) / 64;  // 1 KB loads per page: 19
constexpr int kLatStage = kLatLoads * 64;         // uint4 per stage (tail slots unused)
constexpr int kLatStages = 3;

// Waits until at most n vector memory operations of this wave are outstanding, n <= 20.
__device__ __forceinline__ void wait_vm_upto20(int n) {
#define PSD_W(N) case N: __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70); break;
  switch (n) {
    PSD_W(0) PSD_W(1) PSD_W(2) PSD_W(3) PSD_W(4) PSD_W(5) PSD_W(6) PSD_W(7) PSD_W(8) PSD_W(9)
    PSD_W(10) PSD_W(11) PSD_W(12) PSD_W(13) PSD_W(14) PSD_W(15) PSD_W(16) PSD_W(17)
    PSD_W(18) PSD_W(19)
    default: __builtin_amdgcn_s_waitcnt(0xF70); break;
  }
#undef PSD_W
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4l;

// Four 16-byte LDS reads in one asm block (with the wait for them), so that the compiler
// does not make them wait for the loads still streaming into other stages.
__device__ __forceinline__ void lds_read4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3,
                                          uint4& x0, uint4& x1, uint4& x2, uint4& x3) {
  u32x4l r0, r1, r2, r3;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
      : "memory");
  x0 = make_uint4(r0.x, r0.y, r0.z, r0.w);
  x1 = make_uint4(r1.x, r1.y, r1.z, r1.w);
  x2 = make_uint4(r2.x, r2.y, r2.z, r2.w);
  x3 = make_uint4(r3.x, r3.y, r3.z, r3.w);
}

__device__ __forceinline__ void lds_read2(uint32_t a0, uint32_t a1, uint4& x0, uint4& x1) {
  u32x4l r0, r1;
  asm volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(a0), "v"(a1)
      : "memory");
  x0 = make_uint4(r0.x, r0.y, r0.z, r0.w);
  x1 = make_uint4(r1.x, r1.y, r1.z, r1.w);
}

// A page's 18 K fragments of the latent tile kernel: every read in one asm block with one
// wait, so that the reads overlap one another and the compiler does not make them wait for
// the loads still streaming into the other slot.
__device__ __forceinline__ void lds_read18(const uint32_t (&ad)[18], uint4 (&x)[18]) {
  u32x4l r0, r1, r2, r3, r4, r5, r6, r7;
  u32x4l r8, r9, r10, r11, r12, r13, r14, r15;
  u32x4l r16, r17;
  asm volatile(
      "ds_read_b128 %0, %18\n\t"
      "ds_read_b128 %1, %19\n\t"
      "ds_read_b128 %2, %20\n\t"
      "ds_read_b128 %3, %21\n\t"
      "ds_read_b128 %4, %22\n\t"
      "ds_read_b128 %5, %23\n\t"
      "ds_read_b128 %6, %24\n\t"
      "ds_read_b128 %7, %25\n\t"
      "ds_read_b128 %8, %26\n\t"
      "ds_read_b128 %9, %27\n\t"
      "ds_read_b128 %10, %28\n\t"
      "ds_read_b128 %11, %29\n\t"
      "ds_read_b128 %12, %30\n\t"
      "ds_read_b128 %13, %31\n\t"
      "ds_read_b128 %14, %32\n\t"
      "ds_read_b128 %15, %33\n\t"
      "ds_read_b128 %16, %34\n\t"
      "ds_read_b128 %17, %35\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
        "=&v"(r7), "=&v"(r8), "=&v"(r9), "=&v"(r10), "=&v"(r11), "=&v"(r12), "=&v"(r13),
        "=&v"(r14), "=&v"(r15), "=&v"(r16), "=&v"(r17)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7]), "v"(ad[8]), "v"(ad[9]), "v"(ad[10]), "v"(ad[11]), "v"(ad[12]),
        "v"(ad[13]), "v"(ad[14]), "v"(ad[15]), "v"(ad[16]), "v"(ad[17])
      : "memory");
  x[0] = make_uint4(r0.x, r0.y, r0.z, r0.w);
  x[1] = make_uint4(r1.x, r1.y, r1.z, r1.w);
  x[2] = make_uint4(r2.x, r2.y, r2.z, r2.w);
  x[3] = make_uint4(r3.x, r3.y, r3.z, r3.w);
  x[4] = make_uint4(r4.x, r4.y, r4.z, r4.w);
  x[5] = make_uint4(r5.x, r5.y, r5.z, r5.w);
  x[6] = make_uint4(r6.x, r6.y, r6.z, r6.w);
  x[7] = make_uint4(r7.x, r7.y, r7.z, r7.w);
  x[8] = make_uint4(r8.x, r8.y, r8.z, r8.w);
  x[9] = make_uint4(r9.x, r9.y, r9.z, r9.w);
  x[10] = make_uint4(r10.x, r10.y, r10.z, r10.w);
  x[11] = make_uint4(r11.x, r11.y, r11.z, r11.w);
  x[12] = make_uint4(r12.x, r12.y, r12.z, r12.w);
  x[13] = make_uint4(r13.x, r13.y, r13.z, r13.w);
  x[14] = make_uint4(r14.x, r14.y, r14.z, r14.w);
  x[15] = make_uint4(r15.x, r15.y, r15.z, r15.w);
  x[16] = make_uint4(r16.x, r16.y, r16.z, r16.w);
  x[17] = make_uint4(r17.x, r17.y, r17.z, r17.w);
}

// A page's 32 V operands of the latent tile kernel, through gfx950's transposing LDS read
// (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element i % 4 of the
// 8-byte reads of lanes 4j + i / 4, j = 0 .. 3. Read k is at byte 32 k from `base`; one
// asm block with one wait, as above.
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2l;
__device__ __forceinline__ void lds_read_tr32(uint32_t base, uint2 (&x)[32]) {
  u32x2l r0, r1, r2, r3, r4, r5, r6, r7;
  u32x2l r8, r9, r10, r11, r12, r13, r14, r15;
  u32x2l r16, r17, r18, r19, r20, r21, r22, r23;
  u32x2l r24, r25, r26, r27, r28, r29, r30, r31;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %32 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %32 offset:32\n\t"
      "ds_read_b64_tr_b16 %2, %32 offset:64\n\t"
      "ds_read_b64_tr_b16 %3, %32 offset:96\n\t"
      "ds_read_b64_tr_b16 %4, %32 offset:128\n\t"
      "ds_read_b64_tr_b16 %5, %32 offset:160\n\t"
      "ds_read_b64_tr_b16 %6, %32 offset:192\n\t"
      "ds_read_b64_tr_b16 %7, %32 offset:224\n\t"
      "ds_read_b64_tr_b16 %8, %32 offset:256\n\t"
      "ds_read_b64_tr_b16 %9, %32 offset:288\n\t"
      "ds_read_b64_tr_b16 %10, %32 offset:320\n\t"
      "ds_read_b64_tr_b16 %11, %32 offset:352\n\t"
      "ds_read_b64_tr_b16 %12, %32 offset:384\n\t"
      "ds_read_b64_tr_b16 %13, %32 offset:416\n\t"
      "ds_read_b64_tr_b16 %14, %32 offset:448\n\t"
      "ds_read_b64_tr_b16 %15, %32 offset:480\n\t"
      "ds_read_b64_tr_b16 %16, %32 offset:512\n\t"
      "ds_read_b64_tr_b16 %17, %32 offset:544\n\t"
      "ds_read_b64_tr_b16 %18, %32 offset:576\n\t"
      "ds_read_b64_tr_b16 %19, %32 offset:608\n\t"
      "ds_read_b64_tr_b16 %20, %32 offset:640\n\t"
      "ds_read_b64_tr_b16 %21, %32 offset:672\n\t"
      "ds_read_b64_tr_b16 %22, %32 offset:704\n\t"
      "ds_read_b64_tr_b16 %23, %32 offset:736\n\t"
      "ds_read_b64_tr_b16 %24, %32 offset:768\n\t"
      "ds_read_b64_tr_b16 %25, %32 offset:800\n\t"
      "ds_read_b64_tr_b16 %26, %32 offset:832\n\t"
      "ds_read_b64_tr_b16 %27, %32 offset:864\n\t"
      "ds_read_b64_tr_b16 %28, %32 offset:896\n\t"
      "ds_read_b64_tr_b16 %29, %32 offset:928\n\t"
      "ds_read_b64_tr_b16 %30, %32 offset:960\n\t"
      "ds_read_b64_tr_b16 %31, %32 offset:992\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6),
        "=&v"(r7), "=&v"(r8), "=&v"(r9), "=&v"(r10), "=&v"(r11), "=&v"(r12), "=&v"(r13),
        "=&v"(r14), "=&v"(r15), "=&v"(r16), "=&v"(r17), "=&v"(r18), "=&v"(r19), "=&v"(r20),
        "=&v"(r21), "=&v"(r22), "=&v"(r23), "=&v"(r24), "=&v"(r25), "=&v"(r26), "=&v"(r27),
        "=&v"(r28), "=&v"(r29), "=&v"(r30), "=&v"(r31)
      : "v"(base)
      : "memory");
  x[0] = make_uint2(r0.x, r0.y);
  x[1] = make_uint2(r1.x, r1.y);
  x[2] = make_uint2(r2.x, r2.y);
  x[3] = make_uint2(r3.x, r3.y);
  x[4] = make_uint2(r4.x, r4.y);
  x[5] = make_uint2(r5.x, r5.y);
  x[6] = make_uint2(r6.x, r6.y);
  x[7] = make_uint2(r7.x, r7.y);
  x[8] = make_uint2(r8.x, r8.y);
  x[9] = make_uint2(r9.x, r9.y);
  x[10] = make_uint2(r10.x, r10.y);
  x[11] = make_uint2(r11.x, r11.y);
  x[12] = make_uint2(r12.x, r12.y);
  x[13] = make_uint2(r13.x, r13.y);
  x[14] = make_uint2(r14.x, r14.y);
  x[15] = make_uint2(r15.x, r15.y);
  x[16] = make_uint2(r16.x, r16.y);
  x[17] = make_uint2(r17.x, r17.y);
  x[18] = make_uint2(r18.x, r18.y);
  x[19] = make_uint2(r19.x, r19.y);
  x[20] = make_uint2(r20.x, r20.y);
  x[21] = make_uint2(r21.x, r21.y);
  x[22] = make_uint2(r22.x, r22.y);
  x[23] = make_uint2(r23.x, r23.y);
  x[24] = make_uint2(r24.x, r24.y);
  x[25] = make_uint2(r25.x, r25.y);
  x[26] = make_uint2(r26.x, r26.y);
  x[27] = make_uint2(r27.x, r27.y);
  x[28] = make_uint2(r28.x, r28.y);
  x[29] = make_uint2(r29.x, r29.y);
  x[30] = make_uint2(r30.x, r30.y);
  x[31] = make_uint2(r31.x, r31.y);
}

template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void attn_latent_kernel(AttnArgs a) {
  constexpr int DQK = 576, DV = 512, NQ = DQK / 32, NC = DV / 16;  // 18 and 32
  __shared__ uint4 stage[kLatStages * kLatStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int p0 = split * a.pps;
  int sel_lp = p0 + lane;
  if (a.sel) sel_lp = a.sel[(int64_t)(s * a.Hkv + g) * a.b_max + min(p0 + lane, a.b_max - 1)];
  const int L = a.lens[s];
  const int n = ceil_div(L, kPage);
  int count = a.sel ? min(a.cnt[s * a.Hkv + g], a.b_max) : n;
  if (count < 0) count = 0;
  if (p0 >= count) return;  // uniform over the workgroup
  const int np = min(a.pps, count - p0);
  int my_lp = 0, my_blk = 0;
  if (lane < np) {
    my_lp = min(max(sel_lp, 0), n - 1);
    my_blk = a.bt[(int64_t)s * a.max_pages + my_lp];
    my_blk = min(max(my_blk, 0), a.num_blocks - 1);
  }

  // this wave's 16 heads' q as B fragments: head r, dims 32c + 8grp .. +8
  const int head = wave * 16 + r;
  const bool hvalid = head < a.G;
  const int64_t qrow = ((int64_t)s * a.Hq + g * a.G + (hvalid ? head : 0)) * DQK;
  uint4 qf[NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c)
    qf[c] = hvalid ? load16(static_cast<const uint16_t*>(a.q) + qrow + 32 * c + 8 * grp)
                   : make_uint4(0, 0, 0, 0);

  // Page loads: instruction i of a page is issued by wave i % WAVES; its lane l fills
  // stage slot 64 i + l = (row, piece) of the padded layout, fetching piece 0 of the row
  // for the pad slot and the tail slots (never read).
  const uint16_t* kb = static_cast<const uint16_t*>(a.k);
  const int my_loads = (kLatLoads - wave + WAVES - 1) / WAVES;
  auto issue = [&](int i, int st) {
    const int blk = __builtin_amdgcn_readlane(my_blk, i);
    const uint16_t* pbase = kb + (int64_t)blk * a.kbs + (int64_t)g * a.khs;
    for (int ins = wave; ins < kLatLoads; ins += WAVES) {
      const int slot = ins * 64 + lane;
      int row = slot / kLatRowPieces, piece = slot - row * kLatRowPieces;
      if (row >= 16) {
        row = 15;
        piece = 0;
      }
      if (piece == kLatRowPieces - 1) piece = 0;
      __builtin_amdgcn_global_load_lds(
          pbase + (int64_t)row * a.kts + piece * 8,
          (__attribute__((address_space(3))) void*)(stage + st * kLatStage + ins * 64), 16, 0,
          0);
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  float4v acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};

  const uint32_t sbase = (uint32_t)(uintptr_t)stage;
  issue(0, 0);
  if (np > 1) issue(1, 1);
  for (int i = 0; i < np; ++i) {
    // page i has landed once only page i + 1's loads of this wave are outstanding
    wait_vm_upto20(i + 1 < np ? my_loads : 0);
    __syncthreads();  // every wave's share of page i is in; page i - 1 is read by all
    if (i + 2 < np) issue(i + 2, (i + 2) % kLatStages);
    const uint32_t st = sbase + (uint32_t)((i % kLatStages) * kLatStage * 16);
    const int lp = __builtin_amdgcn_readlane(my_lp, i);
    const int valid = min(kPage, L - lp * kPage);

    // ---- S^T = K Q^T: K row r, dims 32c + 8grp (piece 4c + grp) ---------------------
    float4v sacc = {0.f, 0.f, 0.f, 0.f};
    const uint32_t krow = st + (uint32_t)(r * kLatRowPieces + grp) * 16;
#pragma unroll
    for (int c0 = 0; c0 < NQ; c0 += 2) {
      uint4 k[2];
      lds_read2(krow + 64 * c0, krow + 64 * (c0 + 1), k[0], k[1]);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[c]), as_bf16x8(qf[c0 + c]),
                                                       sacc, 0, 0, 0);
    }

    // ---- online softmax ------------------------------------------------------------------
    float z[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) z[j] = 4 * grp + j < valid ? sacc[j] * a.sl2 : -INFINITY;
    const float m_loc = wave_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    const float m_new = fmaxf(m_run, m_loc);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? exp2f(m_run - m_new) : 1.f;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = live ? exp2f(z[j] - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum4(p[0] + p[1] + p[2] + p[3]);
    m_run = m_new;
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ph[j] = f2bf(p[j]);
      pl[j] = f2bf(p[j] - __uint_as_float(ph[j] << 16));
    }
    const bf16x8 PP = as_bf16x8(make_uint4(pack2(ph[0], ph[1]), pack2(ph[2], ph[3]),
                                           pack2(pl[0], pl[1]), pack2(pl[2], pl[3])));
    float al[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) al[j] = __shfl(alpha, 4 * grp + j, 64);
    if (__ballot(alpha != 1.f)) {  // skipped once no head's running max moves
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[c][j] *= al[j];
    }

    // ---- O += P V: V rows 4grp + j, piece 16w + r ---------------------------------------
    const uint32_t vrow = st + (uint32_t)((4 * grp) * kLatRowPieces + r) * 16;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint4 x[4];
      lds_read4(vrow + 16 * (0 * kLatRowPieces + 16 * w), vrow + 16 * (1 * kLatRowPieces + 16 * w),
                vrow + 16 * (2 * kLatRowPieces + 16 * w), vrow + 16 * (3 * kLatRowPieces + 16 * w),
                x[0], x[1], x[2], x[3]);
      uint32_t vh[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (4 * grp + j >= valid) x[j] = make_uint4(0u, 0u, 0u, 0u);  // unwritten slots
        vh[j][0] = x[j].x; vh[j][1] = x[j].y; vh[j][2] = x[j].z; vh[j][3] = x[j].w;
      }
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const int wd = cc >> 1;
        const bool hiw = cc & 1;
        uint32_t e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = hiw ? (vh[j][wd] >> 16) : (vh[j][wd] & 0xffffu);
        const uint32_t v01 = pack2(e[0], e[1]), v23 = pack2(e[2], e[3]);
        acc[8 * w + cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            PP, as_bf16x8(make_uint4(v01, v23, v01, v23)), acc[8 * w + cc], 0, 0, 0);
      }
    }
  }

  // ---- partials: rows are heads 4grp + j; tile 8w + cc column r is d = 128w + 8r + cc ---
  const int64_t ubase = (int64_t)s * a.Hq + g * a.G;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = wave * 16 + 4 * grp + j;
    if (hh < a.G) {
      float* dst = a.pacc + ((ubase + hh) * a.nsplit + split) * DV + 8 * r;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<float4*>(dst + 128 * w) =
            make_float4(acc[8 * w][j], acc[8 * w + 1][j], acc[8 * w + 2][j], acc[8 * w + 3][j]);
        *reinterpret_cast<float4*>(dst + 128 * w + 4) =
            make_float4(acc[8 * w + 4][j], acc[8 * w + 5][j], acc[8 * w + 6][j], acc[8 * w + 7][j]);
      }
    }
  }
  if (grp == 0 && hvalid) a.pml[(ubase + head) * a.nsplit + split] = make_float2(m_run, l_run);
}

// ---- latent (MLA-style) attention, one 16-head tile per workgroup ----------------------
//
// The sparse latent step keeps about 200 pages per sequence for 128 query heads. Splitting
// those pages over enough workgroups to fill the GPU, each attending every head, writes
// one 128-head partial per split, as many bytes as the latent rows it read. Here a
// workgroup takes one (sequence, split, 16-head tile); the tiles of one (sequence, split)
// are mapped to one XCD, so that all but the first read of each latent row hit its L2.
// The SUB waves of the workgroup take every SUB-th page of the split, and their states are
// combined in LDS into one partial of 16 heads, so the partials shrink to (splits per
// sequence) x 128 heads x (512 + 2) floats.
//
// Each wave streams its own pages through a private two-slot LDS ring with direct-to-LDS
// loads (page i + 1 in flight while page i is computed; no registers held by loads in
// flight), in the padded row layout of the staged kernel above, and reads its K and V
// fragments from there, each set in one read group with one wait: S^T = K Q^T (18 MFMAs
// 16x16x32 bf16, q of its 16 heads in registers) and O += P V (32 MFMAs; tile c's V
// operand comes from a transposing read: lane (r, grp) gets tokens 4grp .. 4grp+3 of
// column 16c + r).
// Two fp32 values rounded to bf16 (nearest even) and packed, the first in bits 15:0.
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

constexpr int kLatSub = 4;     // waves (page sub-splits) of a tile workgroup

// Waits until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}
constexpr float kLazy = 8.f;   // reference-max slack of the tile kernel's softmax (base 2)

__device__ __forceinline__ int latent_tile_count(const AttnArgs& a) {
  return (a.G + 15) / 16;
}

// LDS of a tile workgroup: the rings (2 pages per wave) and, after the page loop, the
// combine area acc [SUB][16][512] | (m, l) [SUB][16], which overlaps them.
template <int SUB>
constexpr size_t latent_tile_lds() {
  constexpr size_t ring = (size_t)SUB * 2 * kLatStage * 16;
  constexpr size_t comb = (size_t)SUB * 16 * 512 * 4 + SUB * 16 * 8;
  return ring > comb ? ring : comb;
}

template <int SUB>
__global__ __launch_bounds__(64 * SUB) __attribute__((amdgpu_waves_per_eu(1)))
void attn_latent_tile_kernel(AttnArgs a) {
  constexpr int DQK = 576, DV = 512, NQ = DQK / 32, NC = DV / 16;  // 18 and 32
  extern __shared__ uint4 ring[];  // [SUB][2][kLatStage]; later the combine area
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar LDS bases
  const int r = lane & 15, grp = lane >> 4;
  // Workgroup i runs on XCD i % 8: each XCD gets a contiguous range of work items, and
  // the tiles of a (sequence, split) are consecutive items.
  const int tiles = latent_tile_count(a);
  const int N = gridDim.x, wi = blockIdx.x;
  const int idx = (N % 8 == 0) ? (wi % 8) * (N / 8) + wi / 8 : wi;
  const int tile = idx % tiles;
  const int pair = idx / tiles;
  const int split = pair % a.nsplit;
  const int g = (pair / a.nsplit) % a.Hkv, s = pair / a.nsplit / a.Hkv;

  const int L = a.lens[s];
  const int n = ceil_div(L, kPage);
  int count = a.sel ? min(a.cnt[s * a.Hkv + g], a.b_max) : n;
  if (count < 0) count = 0;  // flagged unit: the merge writes NaN
  const int p0 = split * a.pps;
  if (p0 >= count) return;  // uniform over the workgroup, before any barrier
  const int span = min(count - p0, a.pps);
  const int mine = span > wave ? (span - wave + SUB - 1) / SUB : 0;  // <= 64 (plan)

  // lane j holds this wave's j-th page: list entry p0 + wave + SUB j
  int my_lp = 0, my_blk = 0;
  if (lane < mine) {
    const int e = p0 + wave + SUB * lane;
    int lp = a.sel ? a.sel[(int64_t)(s * a.Hkv + g) * a.b_max + e] : e;
    lp = min(max(lp, 0), n - 1);
    my_lp = lp;
    my_blk = min(max(a.bt[(int64_t)s * a.max_pages + lp], 0), a.num_blocks - 1);
  }

  // this wave's 16 heads' q as B fragments: head r, dims 32c + 8grp .. +8
  const int head = tile * 16 + r;  // within the group
  const bool hvalid = head < a.G;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) +
                       ((int64_t)s * a.Hq + g * a.G + (hvalid ? head : 0)) * DQK + 8 * grp;
  uint4 qf[NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c) qf[c] = hvalid ? load16(qb + 32 * c) : make_uint4(0, 0, 0, 0);

  // Page i of this wave into ring slot i & 1: load instruction `ins` fills slots
  // 64 ins + lane = (row, piece) of the padded layout (the pad and tail slots fetch piece
  // 0 of row 15, never read). Past the wave's last page it repeats the last page, so that
  // exactly one page's kLatLoads loads are in flight behind the page being computed.
  uint4* myring = ring + wave * 2 * kLatStage;
  const unsigned char* kb = static_cast<const unsigned char*>(a.k);
  const uint32_t kts_bytes = (uint32_t)(a.kts * 2);  // a page's rows span < 32 KB
  // byte offsets within a page of this lane's piece in each staging load (loop-invariant)
  uint32_t soff[kLatLoads];
#pragma unroll
  for (int ins = 0; ins < kLatLoads; ++ins) {
    const int at = ins * 64 + lane;
    int row = at / kLatRowPieces, piece = at - row * kLatRowPieces;
    if (row >= 16) {
      row = 15;
      piece = 0;
    }
    if (piece == kLatRowPieces - 1) piece = 0;
    soff[ins] = (uint32_t)row * kts_bytes + (uint32_t)piece * 16u;
  }
  auto page_base = [&](int i) {
    const int blk = __builtin_amdgcn_readlane(my_blk, min(i, mine - 1));
    return kb + ((int64_t)blk * a.kbs + (int64_t)g * a.khs) * 2;
  };
  auto issue = [&](int i) {
    const unsigned char* pbase = page_base(i);
    uint4* slot = myring + (i & 1) * kLatStage;
#pragma unroll
    for (int ins = 0; ins < kLatLoads; ++ins)
      __builtin_amdgcn_global_load_lds(pbase + soff[ins],
                                       (__attribute__((address_space(3))) void*)(slot + ins * 64),
                                       16, 0, 0);
  };

  float m_run = -INFINITY, l_run = 0.f;
  float4v acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};

  const uint32_t rbase = (uint32_t)(uintptr_t)myring;
  // S^T = K Q^T for page i, once its loads have landed: K row r, dims 32c + 8grp
  // (piece 4c + grp), scaled to base-2 exponents and masked past the sequence
  auto scores = [&](int i, float (&z)[4]) {
    issue(i + 1);
    wait_vm_n<kLatLoads>();  // page i has landed: only page i + 1's loads are in flight
    const uint32_t st = rbase + (uint32_t)((i & 1) * kLatStage * 16);
    const int valid = min(kPage, L - __builtin_amdgcn_readlane(my_lp, i) * kPage);
    // all 18 K fragments in one read group, then three independent accumulation chains
    // over the 18 steps, summed at the end
    float4v s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0;
    const uint32_t krow = st + (uint32_t)(r * kLatRowPieces + grp) * 16;
    uint32_t kad[NQ];
    uint4 k[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) kad[c] = krow + 64 * c;
    lds_read18(kad, k);
#pragma unroll
    for (int c = 0; c < NQ; c += 3) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[c]), as_bf16x8(qf[c]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[c + 1]), as_bf16x8(qf[c + 1]), s1, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(k[c + 2]), as_bf16x8(qf[c + 2]), s2, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      z[j] = 4 * grp + j < valid ? (s0[j] + s1[j] + s2[j]) * a.sl2 : -INFINITY;
  };
  // the page's weights against the current reference, then O += P V (V rows 4grp + j at
  // piece 16w + r)
  auto accumulate = [&](int i, const float (&z)[4]) {
    const uint32_t st = rbase + (uint32_t)((i & 1) * kLatStage * 16);
    const int valid = min(kPage, L - __builtin_amdgcn_readlane(my_lp, i) * kPage);
    const bool live = m_run != -INFINITY;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = live ? exp2f(z[j] - m_run) : 0.f;
    l_run += wave_sum4(p[0] + p[1] + p[2] + p[3]);
    // P as bf16 hi + lo parts (hardware round to nearest even, two values per convert)
    const uint32_t h01 = pk_bf16(p[0], p[1]), h23 = pk_bf16(p[2], p[3]);
    const uint32_t l01 = pk_bf16(p[0] - bf_lo(h01), p[1] - bf_hi(h01));
    const uint32_t l23 = pk_bf16(p[2] - bf_lo(h23), p[3] - bf_hi(h23));
    const bf16x8 PP = as_bf16x8(make_uint4(h01, h23, l01, l23));
    // V as the B operand straight from LDS: the transposing read of tile c gives lane
    // (r, grp) the tokens 4grp .. 4grp+3 of column 16c + r (lanes s of a 16-lane group
    // read row 4grp + s/4 at columns 16c + 4(s % 4))
    const uint32_t vtr = st + (uint32_t)((4 * grp + (r >> 2)) * kLatRowPieces) * 16 + 8 * (r & 3);
    uint2 vt[NC];
    lds_read_tr32(vtr, vt);
    if (valid < kPage) {  // uniform: only a sequence's last page has unwritten slots
      const uint32_t m01 = (4 * grp + 0 < valid ? 0xffffu : 0u) | (4 * grp + 1 < valid ? 0xffff0000u : 0u);
      const uint32_t m23 = (4 * grp + 2 < valid ? 0xffffu : 0u) | (4 * grp + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        vt[c].x &= m01;
        vt[c].y &= m23;
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          PP, as_bf16x8(make_uint4(vt[c].x, vt[c].y, vt[c].x, vt[c].y)), acc[c], 0, 0, 0);
  };

  // Online softmax with a lazily moved reference: a head's weights are taken relative to
  // a reference m_run that moves (and the accumulators with it) only when the page max
  // exceeds it by more than kLazy (base-2 units), so every weight stays below 2^kLazy,
  // far inside fp32, and the weights and the normaliser share one reference. The move is
  // the outer step below; the inner loop never touches the accumulators outside the
  // matrix cores (a conditional rescale inside it made the compiler copy all 128
  // accumulators out of and back into the AGPRs on every page).
  if (mine > 0) {
    issue(0);
  }
  int i = 0;
  float z[4];
  bool have = false;  // z holds page i's scores already
  while (i < mine) {
    if (!have) scores(i, z);
    {
      const float m_loc = wave_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
      const float m_new = m_loc > m_run + kLazy ? m_loc : m_run;  // -inf + kLazy is -inf
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
      float al[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) al[j] = __shfl(alpha, 4 * grp + j, 64);
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[c][j] *= al[j];
    }
    accumulate(i, z);
    have = false;
    for (++i; i < mine; ++i) {
      scores(i, z);
      const float m_loc = wave_max4(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
      if (__ballot(m_loc > m_run + kLazy)) {
        have = true;
        break;
      }
      accumulate(i, z);
    }
  }

  // ---- the SUB waves' states -> one partial of 16 heads for this split -----------------
  // acc rows are heads 4grp + j; tile c column r is d = 16c + r. The combine
  // area overlaps the rings: the trailing repeat of the last page must land, and every
  // wave must be past its pages, first.
  wait_vm_upto20(0);
  __syncthreads();
  float* tsh = reinterpret_cast<float*>(ring);
  float2* tml = reinterpret_cast<float2*>(tsh + SUB * 16 * DV);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float* dst = tsh + (wave * 16 + 4 * grp + j) * DV + r;
#pragma unroll
    for (int c = 0; c < NC; ++c) dst[16 * c] = acc[c][j];
  }
  if (grp == 0) tml[wave * 16 + r] = make_float2(m_run, l_run);
  __syncthreads();
  const int64_t ubase = (int64_t)s * a.Hq + g * a.G;
  for (int t = threadIdx.x; t < 16 * (DV / 4); t += 64 * SUB) {
    const int h = t / (DV / 4), d4 = t - h * (DV / 4);
    if (tile * 16 + h >= a.G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < SUB; ++w) M = fmaxf(M, tml[w * 16 + h].x);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < SUB; ++w) {
      const float2 ml = tml[w * 16 + h];
      const float wt = ml.x == -INFINITY ? 0.f : exp2f(ml.x - M);  // a wave without pages
      const float4 x = *reinterpret_cast<const float4*>(tsh + (w * 16 + h) * DV + 4 * d4);
      o.x += x.x * wt;
      o.y += x.y * wt;
      o.z += x.z * wt;
      o.w += x.w * wt;
      l += ml.y * wt;
    }
    const int64_t row = (ubase + tile * 16 + h) * a.nsplit + split;
    reinterpret_cast<float4*>(a.pacc + row * DV)[d4] = o;
    if (d4 == 0) a.pml[row] = make_float2(M, l);
  }
}

template <int NT>
__device__ __forceinline__ float block_reduce(float x, float* red, bool is_max) {
  constexpr int NW = NT / 64;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float y = __shfl_xor(x, off, 64);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x = is_max ? fmaxf(x, red[i]) : x + red[i];
  __syncthreads();
  return x;
}

// One workgroup per (query head, sequence). The split weights 2^(m_i - M) are computed
// in parallel; the weighted sum of the partial accumulators is cut into slices of splits
// (thread = (slice, 4 dims)), so that many independent loads are in flight, and the
// slices are summed through LDS.
template <int NT>
__global__ __launch_bounds__(NT) void lse_merge_kernel(MergeArgs a) {
  extern __shared__ float sh[];  // weights [nsplit] | slice sums [slices][Dv]
  __shared__ float red[NT / 64];
  const int h = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int g = h / a.G;
  const int64_t row = ((int64_t)s * a.Hq + h) * a.nsplit;
  const int v4 = a.Dv / 4;
  const int slices = NT / v4;
  const int slice = tid / v4, c = tid - slice * v4;
  const float4* acc = reinterpret_cast<const float4*>(a.pacc) + row * v4 + c;
  // The first (m, l) of each thread and its slice's first PF partial rows are requested
  // together with the length and the count, before the number of splits is known: the
  // workspace holds nsplit entries per row, and entries past the unit's splits are never
  // used. The sums below run in the same order either way.
  constexpr int PF = 4;
  const float2 ml0 = tid < a.nsplit ? a.pml[row + tid] : make_float2(-INFINITY, 0.f);
  float4 xp[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int i = slice + k * slices;
    xp[k] = (slice < slices && i < a.nsplit) ? acc[(int64_t)i * v4]
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int L = a.lens[s];
  const int n = ceil_div(L, kPage);
  const int count = a.cnt ? min(a.cnt[s * a.Hkv + g], a.b_max) : n;
  float* out = a.out + ((int64_t)s * a.Hq + h) * a.Dv;
  if (count <= 0) {
    for (int d = tid; d < a.Dv; d += NT) out[d] = __builtin_nanf("");
    return;
  }
  const int nsp = ceil_div(count, a.pps);
  float m = -INFINITY;
  if (tid < nsp) m = fmaxf(m, ml0.x);
  for (int i = tid + NT; i < nsp; i += NT) m = fmaxf(m, a.pml[row + i].x);
  const float M = block_reduce<NT>(m, red, true);
  float* wts = sh;
  float l = 0.f;
  for (int i = tid; i < nsp; i += NT) {
    const float2 ml = i == tid ? ml0 : a.pml[row + i];
    const float w = exp2f(ml.x - M);
    wts[i] = w;
    l += ml.y * w;
  }
  const float inv = 1.f / block_reduce<NT>(l, red, false);  // also publishes wts
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (slice < slices) {
    auto add = [&](const float4& x, int i) {
      const float w = wts[i];
      o.x += x.x * w;
      o.y += x.y * w;
      o.z += x.z * w;
      o.w += x.w * w;
    };
#pragma unroll
    for (int k = 0; k < PF; ++k)
      if (slice + k * slices < nsp) add(xp[k], slice + k * slices);
#pragma unroll 4
    for (int i = slice + PF * slices; i < nsp; i += slices) add(acc[(int64_t)i * v4], i);
  }
  float4* part = reinterpret_cast<float4*>(sh + ((a.nsplit + 3) & ~3));
  if (slices > 1) {
    if (slice < slices) part[slice * v4 + c] = o;
    __syncthreads();
    if (tid < v4) {
      for (int j = 1; j < slices; ++j) {
        const float4 x = part[j * v4 + tid];
        o.x += x.x;
        o.y += x.y;
        o.z += x.z;
        o.w += x.w;
      }
    }
  }
  if (tid < v4)
    reinterpret_cast<float4*>(out)[tid] = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

template <bool BF16, int DQK, int DV, bool TIER = false>
hipError_t launch_attn(const AttnArgs& a, dim3 grid, int waves, hipStream_t st) {
  // occupancy target per variant: the smallest register budget that does not spill
  constexpr int W1 = DQK > 128 ? 1 : (BF16 ? PSD_ATTN_W1 : 2);
  constexpr int W2 = DQK > 128 ? 1 : 2;
  constexpr bool KT = BF16 && DQK == 128;  // K through an LDS tile per wave
  constexpr size_t T = KT ? kKTileBytes : 0;
  if constexpr (TIER) {  // value tier: groups of up to 16 heads (one wave)
    if (waves != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<BF16, DQK, DV, 1, W1, 0, true, KT>), grid, dim3(64), T, st,
                       a, 0, (int)T);
    return hipGetLastError();
  }
  if (waves == 1) {
    hipLaunchKernelGGL((attn_kernel<BF16, DQK, DV, 1, W1, 0, false, KT>), grid, dim3(64), T, st,
                       a, 0, (int)T);
  } else if (waves == 2) {
    hipLaunchKernelGGL((attn_kernel<BF16, DQK, DV, 2, W2, 0, false, KT>), grid, dim3(128), 2 * T,
                       st, a, 0, (int)T);
  } else {
    hipLaunchKernelGGL((attn_kernel<BF16, DQK, DV, 8, 1, 0, false, KT>), grid, dim3(64 * waves),
                       waves * T, st, a, 0, (int)T);
  }
  return hipGetLastError();
}

// `lds`: the closing combine's bytes; at bf16, D = 128 the waves' K tiles are placed by
// ktile_place.
template <bool BF16, int D, int NW = PSD_ATTN_UNIT_WAVES, bool TIER = false>
hipError_t launch_unit(const Geo& g, const AttnArgs& a, dim3 grid, size_t lds, hipStream_t st) {
  constexpr bool KT = BF16 && D == 128;
  auto kern = &attn_kernel<BF16, D, D, 1, (NW + 3) / 4, NW, TIER, KT>;
  KTilePlace kp{0, 0, lds};
  if (KT) kp = ktile_place(g, NW, lds);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kp.end);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(64 * NW), kp.end, st, a, (int)kp.off, (int)kp.stride);
  return hipGetLastError();
}

hipError_t launch_latent_tiles(const AttnArgs& a, int workgroups, hipStream_t st) {
  constexpr size_t lds = latent_tile_lds<kLatSub>();
  static_assert(lds <= 160 * 1024, "LDS of a tile workgroup");
  auto kern = &attn_latent_tile_kernel<kLatSub>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(workgroups), dim3(64 * kLatSub), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_latent(const AttnArgs& a, dim3 grid, int waves, hipStream_t st) {
  switch (waves) {
    case 1: hipLaunchKernelGGL(attn_latent_kernel<1>, grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL(attn_latent_kernel<2>, grid, dim3(128), 0, st, a); break;
    case 3: hipLaunchKernelGGL(attn_latent_kernel<3>, grid, dim3(192), 0, st, a); break;
    case 4: hipLaunchKernelGGL(attn_latent_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 5: hipLaunchKernelGGL(attn_latent_kernel<5>, grid, dim3(320), 0, st, a); break;
    case 6: hipLaunchKernelGGL(attn_latent_kernel<6>, grid, dim3(384), 0, st, a); break;
    case 7: hipLaunchKernelGGL(attn_latent_kernel<7>, grid, dim3(448), 0, st, a); break;
    default: hipLaunchKernelGGL(attn_latent_kernel<8>, grid, dim3(512), 0, st, a); break;
  }
  return hipGetLastError();
}

// The split-K partials' merge (log-sum-exp weights), one workgroup per (sequence, query
// head); `cnt` nullptr for the dense walk.
hipError_t launch_split_merge(const Geo& g, const DecodePlan& p, const AttnArgs& a,
                              const int32_t* lens, const int32_t* cnt, int b_max, float* out,
                              hipStream_t st) {
  MergeArgs m{lens, cnt, a.pacc, a.pml, out, g.Hq, g.Hkv, g.G, p.pps, p.nsplit, g.Dv, b_max};
  // wider workgroups when there are many splits to combine
  const int nt = p.nsplit > 32 ? 1024 : 256;
  const size_t lds = ((p.nsplit + 3) & ~3) * sizeof(float) + (size_t)nt * 4 * sizeof(float);
  hipError_t e;
  if (nt == 1024) {
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lse_merge_kernel<1024>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) !=
        hipSuccess)
      return e;
    hipLaunchKernelGGL(lse_merge_kernel<1024>, dim3(g.Hq, g.B), dim3(1024), lds, st, m);
  } else {
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lse_merge_kernel<256>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)) !=
        hipSuccess)
      return e;
    hipLaunchKernelGGL(lse_merge_kernel<256>, dim3(g.Hq, g.B), dim3(256), lds, st, m);
  }
  return hipGetLastError();
}

}  // namespace

bool plan_decode(const Geo& g, int max_pages_attended, bool dense, DecodePlan* p) {
  if (max_pages_attended < 1) return false;
  p->waves = (g.G + 15) / 16;
  const int64_t units = (int64_t)g.B * g.Hkv;
  p->unit = 0;
  p->latent_tiles = 0;
  if (g.G <= 16 && g.D <= 128 && (units >= PSD_ATTN_UNIT_MIN || small_units(g)) &&
      (!dense || PSD_ATTN_UNIT_DENSE)) {
    // one workgroup per unit, its waves the splits, combined in LDS: no partials. fp32 at
    // D = 128 takes 8 waves: its 16-wave build spills at the 128-VGPR budget and was
    // measured to give wrong outputs for two of every four heads, while the 8-wave build
    // (176 VGPRs, no spill) of the same body is exact
    p->unit = (g.dtype != 1 && g.D > 64) ? 8 : PSD_ATTN_UNIT_WAVES;
    p->pps = (max_pages_attended + p->unit - 1) / p->unit;
    p->nsplit = 1;
    p->off_ml = 0;
    p->bytes = 256;
    return true;
  }
  if (!dense && g.D == 576 && g.Dv == 512 && g.dtype == 1) {
    // latent tile plan: (sequence, split, 16-head tile) workgroups of kLatSub waves, about
    // one per CU; each wave takes at most 64 of its split's pages
    const int64_t tiles = (g.G + 15) / 16;
    int64_t ns = (kComputeUnits + units * tiles - 1) / (units * tiles);
    ns = ns < 1 ? 1 : ns;
    const int64_t cap = 64 * kLatSub;
    if ((max_pages_attended + ns - 1) / ns > cap) ns = (max_pages_attended + cap - 1) / cap;
    if (ns > max_pages_attended) ns = max_pages_attended;
    p->latent_tiles = (int)tiles;
    p->nsplit = (int)ns;
    p->pps = (int)((max_pages_attended + ns - 1) / ns);
    const size_t parts = (size_t)g.B * g.Hq * p->nsplit;
    p->off_ml = (parts * g.Dv * sizeof(float) + 255) / 256 * 256;
    p->bytes = p->off_ml + parts * sizeof(float2) + 256;
    return true;
  }
  // Aim for PSD_ATTN_TARGET single-wave workgroups (fewer, larger ones for many-head
  // groups).
  const int64_t target =
      p->waves > 1 ? PSD_ATTN_TARGET_WIDE : (dense ? PSD_ATTN_TARGET_DENSE : PSD_ATTN_TARGET);
  int64_t pps = (units * max_pages_attended + target - 1) / target;
  const int64_t lo = p->waves > 1 ? 4 : 1;
  pps = pps < lo ? lo : (pps > 64 ? 64 : pps);
  p->pps = (int)pps;
  p->nsplit = (max_pages_attended + p->pps - 1) / p->pps;
  if (p->nsplit > kMaxSplits) return false;  // the merge keeps one weight per split in LDS
  const size_t parts = (size_t)g.B * g.Hq * p->nsplit;
  p->off_ml = (parts * g.Dv * sizeof(float) + 255) / 256 * 256;
  p->bytes = p->off_ml + parts * sizeof(float2) + 256;
  return true;
}

hipError_t launch_decode(const Geo& g, const DecodePlan& p, const void* q, const void* k,
                         const void* v, const int32_t* bt, const int32_t* lens,
                         const int32_t* sel, const int32_t* cnt, int b_max, float scale,
                         float* out, void* ws, hipStream_t st) {
  const AttnArgs a = make_attn_args(g, p, q, k, v, bt, lens, sel, cnt, b_max, scale, out, ws);
  const dim3 grid(p.nsplit, g.Hkv, g.B);
  hipError_t e;
  const bool bf = g.dtype == 1;
  if (p.unit) {
    const size_t lds = unit_combine_lds(g);
    const dim3 ugrid(g.Hkv, g.B);
    if (g.D == 64)
      return bf ? launch_unit<true, 64>(g, a, ugrid, lds, st)
                : launch_unit<false, 64>(g, a, ugrid, lds, st);
    if (bf) return launch_unit<true, 128>(g, a, ugrid, lds, st);
    // fp32 D = 128 is built for 8-wave workgroups only (plan_decode)
    return p.unit == 8 ? launch_unit<false, 128, 8>(g, a, ugrid, lds, st) : hipErrorInvalidValue;
  }
  if (g.D == 64)
    e = bf ? launch_attn<true, 64, 64>(a, grid, p.waves, st)
           : launch_attn<false, 64, 64>(a, grid, p.waves, st);
  else if (g.D == 128)
    e = bf ? launch_attn<true, 128, 128>(a, grid, p.waves, st)
           : launch_attn<false, 128, 128>(a, grid, p.waves, st);
  else if (p.latent_tiles && bf && k == v && g.kbs == g.vbs && g.kts == g.vts && g.khs == g.vhs)
    e = launch_latent_tiles(a, (int)((int64_t)g.B * g.Hkv * p.nsplit * p.latent_tiles), st);
  else if (bf && k == v && g.kbs == g.vbs && g.kts == g.vts && g.khs == g.vhs)
    e = launch_latent(a, grid, p.waves, st);
  else
    e = bf ? launch_attn<true, 576, 512>(a, grid, p.waves, st)
           : launch_attn<false, 576, 512>(a, grid, p.waves, st);
  if (e != hipSuccess) return e;
  return launch_split_merge(g, p, a, lens, sel ? cnt : nullptr, b_max, out, st);
}

hipError_t launch_decode_tiered(const Geo& g, const DecodePlan& p, const void* q, const void* k,
                                const void* v, const void* hot_k, const void* hot,
                                const int32_t* vslot, const int32_t* bt, const int32_t* lens,
                                const int32_t* sel, const int32_t* cnt, int b_max, float scale,
                                float* out, void* ws, hipStream_t st) {
  if (p.latent_tiles || g.D != g.Dv || (g.D != 64 && g.D != 128) || g.G > 16)
    return hipErrorInvalidValue;
  AttnArgs a = make_attn_args(g, p, q, k, v, bt, lens, sel, cnt, b_max, scale, out, ws);
  a.vslot = vslot;
  a.hot = hot;
  a.hot_k = hot_k;
  const bool bf = g.dtype == 1;
  hipError_t e;
  if (p.unit) {
    const size_t lds = unit_combine_lds(g);
    const dim3 ugrid(g.Hkv, g.B);
    if (g.D == 64)
      return bf ? launch_unit<true, 64, PSD_ATTN_UNIT_WAVES, true>(g, a, ugrid, lds, st)
                : launch_unit<false, 64, PSD_ATTN_UNIT_WAVES, true>(g, a, ugrid, lds, st);
    if (bf) return launch_unit<true, 128, PSD_ATTN_UNIT_WAVES, true>(g, a, ugrid, lds, st);
    return p.unit == 8 ? launch_unit<false, 128, 8, true>(g, a, ugrid, lds, st)
                       : hipErrorInvalidValue;
  }
  const dim3 grid(p.nsplit, g.Hkv, g.B);
  if (g.D == 64)
    e = bf ? launch_attn<true, 64, 64, true>(a, grid, p.waves, st)
           : launch_attn<false, 64, 64, true>(a, grid, p.waves, st);
  else
    e = bf ? launch_attn<true, 128, 128, true>(a, grid, p.waves, st)
           : launch_attn<false, 128, 128, true>(a, grid, p.waves, st);
  if (e != hipSuccess) return e;
  return launch_split_merge(g, p, a, lens, sel ? cnt : nullptr, b_max, out, st);
}

}  // namespace psd
