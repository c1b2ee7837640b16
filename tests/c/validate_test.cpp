// Host validation of the ISD library (strided_verify_propose_amd/csrc/isd_validate.cpp),
// built alone -- no HIP -- under the address and undefined-behaviour sanitizers:
//   * valid calls fill their launch descriptions, and every scratch region the
//     description points at lies inside the caller's workspace;
//   * each documented error returns its status with a message;
//   * a deterministic fuzz over every entry point's integer arguments (extremes
//     included) runs without undefined behaviour, and a call either fails or yields a
//     workspace carve-up inside the workspace it asked for.
// Exit status 0 when every check holds.
#include <limits.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "validate.h"

using namespace isd;

static int fails = 0;
#define CHECK(cond)                                                       \
  do {                                                                    \
    if (!(cond)) {                                                        \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__);   \
      ++fails;                                                            \
    }                                                                     \
  } while (0)

// device pointers are never touched here: fake addresses with the right alignment
static void* const P = reinterpret_cast<void*>(0x100000);

static bool inside(const void* p, size_t bytes, const char* ws, size_t total) {
  const char* c = static_cast<const char*>(p);
  return c >= ws && c + bytes <= ws + total;
}

static void attention_cases() {
  const size_t need = attention_workspace_bytes(64, 4, 32, 8, 128, 4096);
  CHECK(need > 0);
  std::vector<char> ws(16);
  char* base = reinterpret_cast<char*>(0x2000000);
  AttnLaunch a{};
  isd_status st = prepare_attention(ISD_BF16, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 64, 4, 32, 8,
                                    128, 16, 257, 16448, 4096, 0.088f, base, need, &a);
  CHECK(st == ISD_OK);
  CHECK(a.R == 7 && a.G == 4 && a.B == 64);
  const size_t RG = 28;
  CHECK(inside(a.part_o, (size_t)ATTN_MAX_WG * 2 * RG * 128 * 4, base, need));
  CHECK(inside(a.part_ml, (size_t)ATTN_MAX_WG * 2 * RG * 2 * 4, base, need));
  CHECK(prepare_attention(ISD_BF16, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 64, 4, 32, 8, 128, 16,
                          257, 16448, 4096, 0.088f, base, need - 1, &a) == ISD_ERR_WORKSPACE);
  CHECK(prepare_attention(ISD_BF16, nullptr, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 64, 4, 32, 8, 128,
                          16, 257, 16448, 4096, 0.088f, base, need, &a) == ISD_ERR_INVALID_ARG);
  CHECK(strlen(last_error()) > 0);
  CHECK(prepare_attention(ISD_BF16, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 64, 4, 32, 8, 96, 16,
                          257, 16448, 4096, 0.088f, base, need, &a) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_attention(ISD_BF16, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 64, 4, 32, 8, 128, 8,
                          257, 16448, 4096, 0.088f, base, need, &a) == ISD_ERR_UNSUPPORTED);
  // the context bound must fit the page table
  CHECK(prepare_attention(ISD_BF16, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 64, 4, 32, 8, 128, 16,
                          256, 16448, 4096, 0.088f, base, need, &a) == ISD_ERR_INVALID_ARG);
  // 2048 requests x 8 KV heads at 2.2M tokens: the work list's 32-bit cost sum would overflow
  const int big_ctx = 2200000, big_pages = (big_ctx + 7 + 15) / 16;
  const size_t need_big = attention_workspace_bytes(2048, 4, 32, 8, 128, big_ctx);
  CHECK(prepare_attention(ISD_BF16, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 2048, 4, 32, 8, 128, 16,
                          big_pages, 1 << 30, big_ctx, 0.088f, base, need_big, &a) == ISD_ERR_UNSUPPORTED);
  CHECK(strstr(last_error(), "work units") != nullptr);
  // just under the bound passes
  const int ok_ctx = 2000;
  CHECK(prepare_attention(ISD_BF16, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 2048, 4, 32, 8, 128, 16,
                          (ok_ctx + 22) / 16, 1 << 30, ok_ctx, 0.088f, base, need_big, &a) == ISD_OK);
  CHECK(prepare_attention(ISD_F32, P, P, P, P, P, (const int32_t*)P, (const int32_t*)P, P, 1, 2, 4, 1, 64, 16, 9, 9,
                          128, 0.125f, nullptr, 0, &a) == ISD_OK);
  CHECK(a.dtype == 0 && a.part_o == nullptr);
}

static void kv_pages_cases() {
  KvPagesLaunch c{};
  void* k = reinterpret_cast<void*>(0x1000);
  void* v = reinterpret_cast<void*>(0x2000);
  void* kc = reinterpret_cast<void*>(0x3000);
  void* vc = reinterpret_cast<void*>(0x4000);
  CHECK(prepare_kv_pages(ISD_BF16, k, v, kc, vc, 1000, 8, 128, 1, &c) == ISD_OK && c.to_tiles == 1);
  CHECK(prepare_kv_pages(ISD_F32, kc, vc, k, v, 1000, 8, 64, 0, &c) == ISD_OK && c.to_tiles == 0 && c.dtype == 0);
  CHECK(prepare_kv_pages(ISD_BF16, k, v, k, vc, 1000, 8, 128, 1, &c) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_kv_pages(ISD_BF16, k, v, kc, vc, 1000, 8, 80, 1, &c) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_kv_pages(ISD_BF16, k, v, kc, vc, INT_MAX, 65535, 128, 1, &c) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_kv_pages(ISD_BF16, k, nullptr, kc, vc, 10, 8, 128, 1, &c) == ISD_ERR_INVALID_ARG);

  KvSweepLaunch s{};
  const int32_t* pt = reinterpret_cast<const int32_t*>(0x5000);
  const int32_t* cl = reinterpret_cast<const int32_t*>(0x6000);
  uint32_t* cs = reinterpret_cast<uint32_t*>(0x7000);
  CHECK(prepare_kv_sweep(kc, vc, pt, cl, 64, 8, 128, 257, 20000, 4096, cs, &s) == ISD_OK && s.B == 64 &&
        s.max_pages == 257 && s.checksum == cs);
  CHECK(prepare_kv_sweep(kc, vc, pt, cl, 64, 8, 128, 256, 20000, 4096, cs, &s) == ISD_OK);   // exactly full
  CHECK(prepare_kv_sweep(kc, vc, pt, cl, 64, 8, 128, 256, 20000, 4097, cs, &s) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_kv_sweep(kc, vc, pt, cl, 2049, 8, 128, 257, 20000, 4096, cs, &s) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_kv_sweep(kc, vc, pt, cl, 64, 8, 80, 257, 20000, 4096, cs, &s) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_kv_sweep(kc, vc, pt, nullptr, 64, 8, 128, 257, 20000, 4096, cs, &s) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_kv_sweep(kc, vc, pt, cl, 2048, 65535, 128, 1 << 20, 1 << 30, 1 << 24, cs, &s) ==
        ISD_ERR_UNSUPPORTED);
}

static void verify_cases() {
  const size_t need = verify_workspace_bytes(64, 4, 151936);
  char* base = reinterpret_cast<char*>(0x4000000);
  VerifyLaunch v{};
  CHECK(prepare_verify(ISD_BF16, P, P, (const int32_t*)P, (const float*)P, 64, 4, 151936, 1.f, (int32_t*)P,
                       (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, base, need,
                       &v) == ISD_OK);
  CHECK(v.RR == 10 && v.SV == 10 && v.NSUB == 149);
  const size_t rows = 640;
  CHECK(inside(v.cmax, rows * v.SV * 4, base, need));
  CHECK(inside(v.cidx, rows * v.SV * 4, base, need));
  CHECK(inside(v.csub, rows * v.NSUB * 4, base, need));
  CHECK(inside(v.ws, 64 * sizeof(WalkState), base, need));
  CHECK(inside(v.rsub, 64 * (size_t)v.NSUB * 4, base, need));
  CHECK(prepare_verify(ISD_BF16, P, P, (const int32_t*)P, (const float*)P, 64, 4, 151936, 0.f, (int32_t*)P,
                       (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, base, need,
                       &v) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_verify(ISD_BF16, P, P, (const int32_t*)P, (const float*)P, 64, 9, 151936, 1.f, (int32_t*)P,
                       (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, base, need,
                       &v) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_verify(ISD_BF16, P, P, nullptr, (const float*)P, 64, 4, 151936, 1.f, (int32_t*)P, (uint8_t*)P,
                       (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, base, need,
                       &v) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_verify(ISD_BF16, P, P, (const int32_t*)P, (const float*)P, 64, 4, 151936, 1.f, (int32_t*)P,
                       (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, base, need - 1,
                       &v) == ISD_ERR_WORKSPACE);
  // N == 1: no draft ids needed, no draft rows
  CHECK(prepare_verify(ISD_F32, P, P, nullptr, (const float*)P, 3, 1, 1000, 1.f, (int32_t*)P, nullptr, (int32_t*)P,
                       (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, base, verify_workspace_bytes(3, 1, 1000),
                       &v) == ISD_OK);
  CHECK(v.draft == nullptr && v.RR == 1);
  // statistics carried between steps: the draft rows leave the stats pass, and a carried
  // row holds 2 SV + NSUB floats
  char* prev = reinterpret_cast<char*>(0x10000000);
  char* next = reinterpret_cast<char*>(0x20000000);
  CHECK(prepare_verify_carry(ISD_BF16, P, P, (const int32_t*)P, (const float*)P, 64, 4, 151936, 1.f, (int32_t*)P,
                             (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, prev, next,
                             base, need, &v) == ISD_OK);
  CHECK(v.srow0 == 0 && v.snrow == 7 && v.RR == 10 && v.QS == 2 * 10 + 149);
  CHECK((size_t)64 * 3 * v.QS * 4 == verify_carry_bytes(64, 4, 151936));
  CHECK(prepare_verify_carry(ISD_BF16, P, P, (const int32_t*)P, (const float*)P, 64, 4, 151936, 1.f, (int32_t*)P,
                             (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, nullptr,
                             next, base, need, &v) == ISD_OK);
  CHECK(v.snrow == 10 && v.qprev == nullptr);
  CHECK(prepare_verify_carry(ISD_BF16, P, P, (const int32_t*)P, (const float*)P, 64, 4, 151936, 1.f, (int32_t*)P,
                             (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr, prev, prev,
                             base, need, &v) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_verify_carry(ISD_BF16, P, nullptr, (const int32_t*)P, (const float*)P, 64, 4, 151936, 1.f,
                             (int32_t*)P, (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr, nullptr,
                             prev, next, base, need, &v) == ISD_ERR_INVALID_ARG);
}

static void proj_and_lm_head_cases() {
  char* base = reinterpret_cast<char*>(0x8000000);
  ProjLaunch p{};
  const size_t need = proj_workspace_bytes(448, 4096, 4096, 128);
  CHECK(prepare_proj(P, P, P, P, (const uint8_t*)P, P, 448, 4096, 4096, 128, base, need, &p) == ISD_OK);
  CHECK(p.r == 128 && p.gate != nullptr && inside(p.Ybase, (size_t)448 * 4096 * 4, base, need));
  CHECK(inside(p.T, (size_t)448 * 128 * 2, base, need));
  CHECK(prepare_proj(P, P, nullptr, P, (const uint8_t*)P, P, 448, 4096, 4096, 128, base, need, &p) ==
        ISD_ERR_INVALID_ARG);
  CHECK(prepare_proj(P, P, P, P, (const uint8_t*)P, P, 448, 4096, 4096, 64, base, need, &p) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_proj(P, P, P, P, (const uint8_t*)P, P, 448, 4000, 4096, 128, base, need, &p) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_proj(P, P, nullptr, nullptr, nullptr, P, 448, 4096, 4096, 0, nullptr, 0, &p) == ISD_OK);
  CHECK(proj_packed_bytes(4096, 4096, 128) == (size_t)(4096 + 128) * 4096 * 2 + (size_t)4096 * 128 * 2);
  CHECK(prepare_pack_proj(P, nullptr, nullptr, P, 4096, 4096, 128) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_proj_packed(P, P, (const uint8_t*)P, P, 448, 4096, 4096, 0, base, need, &p) == ISD_ERR_INVALID_ARG);
  CHECK(prepare_proj_packed(P, P, (const uint8_t*)P, P, 448, 4096, 4096, 128, base, need, &p) == ISD_OK);
  CHECK(p.Bl == static_cast<const uint16_t*>(P) + (size_t)(4096 + 128) * 4096);
  // gated and base-only calls split alike
  CHECK(proj_ksplit(448, 4096, 4096) == proj_ksplit(448, 4096, 4096));
  CHECK(proj_big_split(448, 12288, 4096) > 0);

  LmhLaunch l{};
  VerifyLaunch v{};
  CHECK(prepare_lm_head(P, P, P, 448, 4096, 151936, &l) == ISD_OK && l.NMINI == 1187 && l.NMS == 1192);
  CHECK(prepare_lm_head(P, P, P, 448, 4096, 151937, &l) == ISD_ERR_UNSUPPORTED);
  const size_t lneed = lm_head_verify_workspace_bytes(64, 4, 151936);
  CHECK(lneed > verify_workspace_bytes(64, 4, 151936));
  CHECK(prepare_lm_head_verify(P, P, P, P, (const int32_t*)P, (const float*)P, 64, 4, 4096, 151936, 1.f,
                               (int32_t*)P, (uint8_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr,
                               nullptr, base, lneed, &l, &v) == ISD_OK);
  CHECK(v.srow0 == 7 && v.snrow == 3 && l.M == 448);
  CHECK(inside(l.marg, (size_t)448 * l.NMS * 4, base, lneed));
  CommitLaunch c{};
  CHECK(prepare_commit((const int32_t*)P, (const int32_t*)P, (const int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr,
                       nullptr, 4, 9, &c) == ISD_ERR_UNSUPPORTED);
  CHECK(prepare_commit((const int32_t*)P, (const int32_t*)P, (const int32_t*)P, nullptr, (int32_t*)P, nullptr,
                       nullptr, 4, 1, &c) == ISD_OK);
}

// ---------------------------------------------------------------- fuzz
static unsigned long long g_state = 0x9E3779B97F4A7C15ull;
static unsigned long long next_u64() {  // splitmix64
  unsigned long long z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int pick() {
  static const int extremes[] = {INT_MIN, -1, 0, 1, 2, 7, 8, 9, 15, 16, 17, 63, 64, 65, 127, 128, 129, 256,
                                 4095, 4096, 65535, 65536, 65537, 151936, 1 << 20, (1 << 20) + 1, INT_MAX};
  const unsigned long long r = next_u64();
  switch (r % 4) {
    case 0: return extremes[(r >> 8) % (sizeof extremes / sizeof extremes[0])];
    case 1: return (int)((r >> 8) % 300);
    case 2: return (int)((r >> 8) % 70000);
    default: return (int)(r >> 32);
  }
}

static void fuzz(int iters) {
  char* base = reinterpret_cast<char*>(0x10000000);
  for (int it = 0; it < iters; ++it) {
    int a0 = pick(), a1 = pick(), a2 = pick(), a3 = pick(), a4 = pick(), a5 = pick(), a6 = pick();
    {
      const size_t need = attention_workspace_bytes(a0, a1, a2, a3, a4, a5);
      AttnLaunch a{};
      const isd_status st = prepare_attention(it % 2 ? ISD_BF16 : ISD_F32, P, P, P, P, P, (const int32_t*)P,
                                              (const int32_t*)P, P, a0, a1, a2, a3, a4, 16, a6, a6, a5, 1.f, base,
                                              need, &a);
      if (st == ISD_OK && a.part_o) CHECK(need > 0 && inside(a.part_ml, 8, base, need));
    }
    {
      KvPagesLaunch c{};
      (void)prepare_kv_pages(ISD_BF16, P, reinterpret_cast<void*>(0x200000), reinterpret_cast<void*>(0x300000),
                             reinterpret_cast<void*>(0x400000), a0, a1, a2, it & 1, &c);
    }
    {
      KvSweepLaunch c{};
      (void)prepare_kv_sweep(P, P, (const int32_t*)P, (const int32_t*)P, a0, a1, it & 1 ? 128 : 64, a2, a0, a1,
                             (uint32_t*)P, &c);
    }
    {
      const size_t need = verify_workspace_bytes(a0, a1, a2);
      VerifyLaunch v{};
      const isd_status st = prepare_verify(ISD_BF16, P, it % 3 ? P : nullptr, (const int32_t*)P, (const float*)P, a0,
                                           a1, a2, 1.f, (int32_t*)P, (uint8_t*)P, (int32_t*)P, (int32_t*)P,
                                           (int32_t*)P, nullptr, nullptr, nullptr, base, need, &v);
      if (st == ISD_OK)
        CHECK(inside(v.rsub, (size_t)v.B * v.NSUB * 4, base, need) &&
              inside(v.csub, (size_t)v.B * v.RR * v.NSUB * 4, base, need));
    }
    {
      const size_t need = proj_workspace_bytes(a0, a1, a2, a3);
      ProjLaunch p{};
      const isd_status st =
          prepare_proj(P, P, P, P, it % 2 ? (const uint8_t*)P : nullptr, P, a0, a1, a2, a3, base, need, &p);
      if (st == ISD_OK && p.ksplit > 1)
        CHECK(inside(p.part, (size_t)p.ksplit * p.M * (p.Nout + p.r) * 4, base, need));
      (void)proj_packed_bytes(a1, a2, a3);
      (void)prepare_proj_packed(P, P, nullptr, P, a0, a1, a2, a3, base, need, &p);
    }
    {
      LmhLaunch l{};
      VerifyLaunch v{};
      (void)prepare_lm_head(P, P, P, a0, a1, a2, &l);
      const size_t need = lm_head_verify_workspace_bytes(a0, a3, a2);
      const isd_status st = prepare_lm_head_verify(P, P, P, P, (const int32_t*)P, (const float*)P, a0, a3, a1, a2,
                                                   1.f, (int32_t*)P, (uint8_t*)P, (int32_t*)P, (int32_t*)P,
                                                   (int32_t*)P, nullptr, nullptr, nullptr, base, need, &l, &v);
      if (st == ISD_OK) CHECK(inside(l.marg, (size_t)l.M * l.NMS * 4, base, need));
      CommitLaunch c{};
      (void)prepare_commit((const int32_t*)P, (const int32_t*)P, (const int32_t*)P, (int32_t*)P, (int32_t*)P,
                           nullptr, nullptr, a0, a1, &c);
    }
  }
}

int main() {
  attention_cases();
  kv_pages_cases();
  verify_cases();
  proj_and_lm_head_cases();
  fuzz(200000);
  if (fails == 0) printf("validate ok\n");
  return fails == 0 ? 0 : 1;
}
