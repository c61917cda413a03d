// Host-side harness for sanitizer builds.  Links the library's host sources
// (argument checks, workspace layout, the decode planner, the encode and
// 8-bit pool layouts) with stub kernel launchers and stub HIP runtime calls,
// then drives every host path, including tables and arguments the checks
// must refuse.  Built with g++ -fsanitize=address,undefined by
// tests/test_sanitize.py; nothing here touches a GPU.  Every host table is
// an exactly sized heap allocation, so a read past it is reported.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "kernels.h"
#include "milo_attn.h"
#include "milo_encode.h"

static int g_fail = 0;
static int g_launches = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #c); \
      ++g_fail;                                                     \
    }                                                               \
  } while (0)

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }

namespace milo {
hipError_t launch_chunk(const ChunkParams& p, int group, hipStream_t, LaunchEvents) {
  ++g_launches;
  EXPECT(group >= 1 && p.n_ranges >= 1 && p.blocks_per_range >= 1 && p.n_qtiles >= 1);
  EXPECT(p.head_dim == 64 || p.head_dim == 128);
  EXPECT((int64_t)p.n_ranges * p.blocks_per_range >= p.max_blocks);
  return hipSuccess;
}
hipError_t launch_merge(const MergeParams& p, int head_dim, hipStream_t) {
  ++g_launches;
  EXPECT(head_dim == 64 || head_dim == 128);
  EXPECT(p.slots >= 1 && p.tail_slot == p.slots - 1 && p.rows_per_unit >= 1);
  return hipSuccess;
}
hipError_t launch_validate(const ValidateParams& p, hipStream_t) {
  ++g_launches;
  EXPECT(p.status != nullptr);
  return hipSuccess;
}
hipError_t launch_read_probe(const void*, size_t, uint32_t*, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
#define MILO_STUB_DECODE(name)                                        \
  hipError_t name(const DecodeParams& p, int group, hipStream_t, LaunchEvents) { \
    ++g_launches;                                                     \
    EXPECT(group >= 1 && group <= 8 && p.batch >= 1);                 \
    return hipSuccess;                                                \
  }
MILO_STUB_DECODE(launch_decode_dt_0_64)
MILO_STUB_DECODE(launch_decode_dt_0_128)
MILO_STUB_DECODE(launch_decode_dt_1_64)
MILO_STUB_DECODE(launch_decode_dt_1_128)
MILO_STUB_DECODE(launch_decode_dt_2_64)
MILO_STUB_DECODE(launch_decode_dt_2_128)
MILO_STUB_DECODE(launch_decode_dt_3_64)
MILO_STUB_DECODE(launch_decode_dt_3_128)
MILO_STUB_DECODE(launch_decode_dt_4_64)
MILO_STUB_DECODE(launch_decode_dt_4_128)
hipError_t launch_rank(const RankParams&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize(const QuantParams&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize_kivi(const QuantParams&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_encode_factors(const EncodeParams&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_encode_spectrum(const EncodeParams&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace milo

namespace {

// A non-null, suitably aligned address that the host code never dereferences.
void* fake(uintptr_t k = 1) { return reinterpret_cast<void*>(k << 16); }

milo_attn_args base_args(int32_t path) {
  milo_attn_args a{};
  a.struct_size = sizeof(milo_attn_args);
  a.dtype = MILO_BF16;
  a.batch = 3;
  a.q_len = path == MILO_PATH_CHUNK ? 17 : 1;
  a.n_q_heads = 28;
  a.n_kv_heads = 4;
  a.head_dim = 128;
  a.scale = 0.088f;
  a.q = fake(1);
  a.pool = fake(2);
  a.blocks = static_cast<const milo_block*>(fake(3));
  a.seq_blocks = static_cast<const int32_t*>(fake(4));
  a.max_blocks_per_seq = 9;
  a.tail_cap = 40;
  a.k_tail = fake(5);
  a.v_tail = fake(6);
  a.tail_len = static_cast<const int32_t*>(fake(7));
  a.out = static_cast<float*>(fake(8));
  a.lse = static_cast<float*>(fake(9));
  a.workspace = fake(10);
  a.workspace_bytes = 1ull << 40;
  return a;
}

void attention_entry_points() {
  for (int32_t path : {MILO_PATH_DECODE, MILO_PATH_CHUNK, MILO_PATH_SHARED}) {
    auto fn = path == MILO_PATH_DECODE ? milo_attn_decode
              : path == MILO_PATH_CHUNK ? milo_attn_chunk
                                        : milo_attn_decode_shared;
    milo_attn_args a = base_args(path);
    const size_t need = milo_attn_workspace_bytes(&a, path);
    EXPECT(need > 0);
    a.workspace_bytes = need;
    const int before = g_launches;
    EXPECT(fn(&a, nullptr) == MILO_OK);
    EXPECT(g_launches == before + 2);   // the attention kernel and the merge
    // every host-checkable fault is refused before any launch
    std::vector<milo_attn_args> bad(16, a);
    bad[0].struct_size = 8;
    bad[1].q = nullptr;
    bad[2].q = reinterpret_cast<const void*>(uintptr_t(3));
    bad[3].n_q_heads = 27;
    bad[4].head_dim = 96;
    bad[5].scale = 1.0f / 0.0f;
    bad[6].workspace_bytes = need - 1;
    bad[7].workspace = reinterpret_cast<void*>(uintptr_t(0x10010));
    bad[8].tail_len = nullptr;
    bad[9].max_blocks_per_seq = -1;
    bad[10].batch = -2;
    bad[11].dtype = 7;
    bad[12].n_q_heads = 4 * 9;          // group size 9
    bad[13].out = nullptr;
    bad[14].q_len = 0;
    bad[15].lse = reinterpret_cast<float*>(uintptr_t(0x10002));
    for (size_t k = 0; k < bad.size(); ++k) {
      const int b0 = g_launches;
      EXPECT(fn(&bad[k], nullptr) != MILO_OK);
      EXPECT(g_launches == b0);
    }
    milo_attn_args empty = a;
    empty.batch = 0;
    EXPECT(fn(&empty, nullptr) == MILO_OK);
  }
  uint64_t status_word = 0;
  milo_attn_args a = base_args(MILO_PATH_DECODE);
  EXPECT(milo_attn_validate(&a, MILO_PATH_DECODE, 20, 1 << 20, &status_word, nullptr) == MILO_OK);
  EXPECT(milo_attn_validate(&a, MILO_PATH_DECODE, -1, 1 << 20, &status_word, nullptr) == MILO_ERR_INVALID);
  a.unit_order = static_cast<const int32_t*>(fake(11));
  a.workspace = nullptr;
  EXPECT(milo_attn_validate(&a, MILO_PATH_DECODE, 20, 1 << 20, &status_word, nullptr) == MILO_ERR_WORKSPACE);
  EXPECT(milo_read_probe(fake(1), 1 << 20, static_cast<uint32_t*>(fake(2)), 64, nullptr) == MILO_OK);
  EXPECT(milo_read_probe(fake(1), 17, static_cast<uint32_t*>(fake(2)), 64, nullptr) == MILO_ERR_INVALID);
}

// The planner on random tables: lists inside the table are planned into a
// permutation; lists that leave it are refused before any descriptor read.
void planner(std::mt19937& rng) {
  for (int trial = 0; trial < 400; ++trial) {
    const int batch = 1 + rng() % 6, hkv = 1 + rng() % 4, mb = rng() % 7;
    const int n_desc = rng() % 20;
    std::vector<milo_block> blocks(n_desc);
    for (auto& b : blocks) {
      b.off = 8 * (rng() % 1000);
      b.n_tok = rng() % 3000 - 5;
      b.ld_tok = 8 * (rng() % 400);
      b.rank_k = rng() % 140 - 4;
      b.rank_v = rng() % 140 - 4;
    }
    std::vector<int32_t> sb(batch + 1);
    bool inside = true;
    sb[0] = rng() % 3;
    for (int i = 0; i < batch; ++i) sb[i + 1] = sb[i] + rng() % (mb + 2);
    for (int i = 0; i <= batch; ++i) inside = inside && sb[i] <= n_desc;
    std::vector<int32_t> tail(batch);
    for (auto& t : tail) t = rng() % 300 - 3;
    const int64_t units = (int64_t)batch * hkv * (mb + 1);
    std::vector<int32_t> order(units);
    const milo_status st = milo_attn_plan_decode(n_desc ? blocks.data() : nullptr, n_desc, sb.data(),
                                                 (rng() & 1) ? tail.data() : nullptr, batch, hkv, mb, 128,
                                                 order.data());
    if (!inside) {
      EXPECT(st == MILO_ERR_INVALID);
      continue;
    }
    EXPECT(st == MILO_OK);
    std::vector<char> seen(units, 0);
    for (int32_t u : order) {
      EXPECT(u >= 0 && u < units);
      if (u >= 0 && u < units) {
        EXPECT(!seen[u]);
        seen[u] = 1;
      }
    }
  }
  std::vector<int32_t> order(8);
  std::vector<int32_t> sb{0, 0};
  EXPECT(milo_attn_plan_decode(nullptr, 0, sb.data(), nullptr, 1, 1, 0, 128, order.data()) == MILO_OK);
  EXPECT(milo_attn_plan_decode(nullptr, 5, sb.data(), nullptr, 1, 1, 0, 128, order.data()) == MILO_ERR_INVALID);
}

void layouts(std::mt19937& rng) {
  for (int trial = 0; trial < 200; ++trial) {
    const int nb = rng() % 12, hkv = 1 + rng() % 4, d = (rng() & 1) ? 64 : 128;
    std::vector<int32_t> nt(nb), rk(nb), rv(nb);
    for (int b = 0; b < nb; ++b) {
      nt[b] = rng() % 2100;
      rk[b] = rng() % (d + 1);
      rv[b] = rng() % (d + 1);
    }
    std::vector<milo_block> out(nb);
    int64_t elems = -1;
    const milo_status st = milo_encode_layout(nb ? nt.data() : nullptr, nb ? rk.data() : nullptr,
                                              nb ? rv.data() : nullptr, nb, hkv, d,
                                              nb ? out.data() : nullptr, &elems);
    EXPECT(st == MILO_OK);
    if (st != MILO_OK) continue;
    int64_t end = 0;
    for (int b = 0; b < nb; ++b) {
      EXPECT(out[b].n_tok == nt[b] && out[b].ld_tok >= nt[b] && out[b].ld_tok % 8 == 0 && out[b].off % 8 == 0);
      end = std::max<int64_t>(end, out[b].off + (int64_t)hkv * (rk[b] + rv[b]) * (out[b].ld_tok + d));
    }
    EXPECT(elems >= end);
    std::vector<milo_block> q8(nb);
    int64_t bytes = -1;
    EXPECT(milo_quant_layout(nb ? out.data() : nullptr, nb, hkv, d, nb ? q8.data() : nullptr, &bytes) == MILO_OK);
    for (int b = 0; b < nb; ++b) EXPECT(q8[b].off % 16 == 0 && q8[b].ld_tok % 64 == 0 && q8[b].off < bytes + 1);
    for (int bits = 2; bits <= 4; bits += 2) {
      std::vector<milo_block> kv(nb);
      int64_t kbytes = -1;
      EXPECT(milo_kivi_layout(nb ? out.data() : nullptr, nb, hkv, d, bits, nb ? kv.data() : nullptr, &kbytes) ==
             MILO_OK);
      for (int b = 0; b < nb; ++b) EXPECT(kv[b].off % 16 == 0 && kv[b].ld_tok % 64 == 0 && kv[b].off < kbytes + 1);
    }
  }
  int32_t one = 5;
  milo_block ob{};
  int64_t e = 0;
  EXPECT(milo_encode_layout(&one, &one, &one, 1, 1, 0, &ob, &e) != MILO_OK);    // head_dim
  EXPECT(milo_encode_layout(&one, &one, &one, -1, 1, 64, &ob, &e) != MILO_OK);
  one = 200;
  EXPECT(milo_encode_layout(&one, &one, &one, 1, 1, 64, &ob, &e) != MILO_OK);   // rank past head_dim
}

}  // namespace

int main() {
  std::mt19937 rng(12345);
  attention_entry_points();
  planner(rng);
  layouts(rng);
  std::printf("host harness: %d launches, %d failed expectations\n", g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}
