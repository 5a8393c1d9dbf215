// Drives every entry point of the C ABI through its host-side argument
// checks (valid calls reach the stub launchers, invalid ones must return the
// documented status without reaching them), with host arrays sized exactly
// as the ABI promises, so that AddressSanitizer sees any read past them.
// Prints "ok <n>" and exits 0 when every expectation holds.
#include <cstdio>
#include <cstring>
#include <memory>
#include <string>
#include <thread>
#include <vector>

#include "ulysses.h"

extern int g_launches;

namespace {

int g_fail = 0, g_checks = 0;
const uintptr_t kFake = 0x7f0000001000ull;  // never dereferenced: the launchers are stubs

void* fake(int i = 0) { return reinterpret_cast<void*>(kFake + 4096 * uintptr_t(i)); }

void expect(bool cond, const char* what) {
  ++g_checks;
  if (!cond) {
    ++g_fail;
    std::fprintf(stderr, "FAIL: %s (last error: %s)\n", what, uly_last_error());
  }
}

// an exactly sized heap array of n fake device pointers
std::unique_ptr<void*[]> ptrs(int n) {
  std::unique_ptr<void*[]> a(new void*[n]);
  for (int i = 0; i < n; ++i) a[i] = fake(i);
  return a;
}

void permutes() {
  for (int P : {1, 4, 64}) {
    auto sh = ptrs(P);
    const int before = g_launches;
    expect(ulysses_pack(sh.get(), P, 256, 8 * P, 64, ULY_BF16, P - 1, fake(99), nullptr) == ULY_OK, "pack ok");
    expect(ulysses_unpack(fake(99), P, 256, 8 * P, 128, ULY_F32, 0, sh.get(), nullptr) == ULY_OK, "unpack ok");
    expect(ulysses_pack_heads(sh.get(), P, 10, 3, 64, ULY_BF16, 1, 2, fake(99), nullptr) == ULY_OK, "heads ok");
    expect(ulysses_unpack_heads(fake(99), P, 10, 3, 64, ULY_BF16, 0, 3, sh.get(), nullptr) == ULY_OK, "unheads ok");
    expect(ulysses_pack_qkv(sh.get(), P, 16, 4 * P, P, 128, ULY_BF16, 0, fake(1), fake(2), fake(3), nullptr) == ULY_OK,
           "pack_qkv ok");
    expect(ulysses_unpack_qkv(fake(1), fake(2), fake(3), P, 16, 4 * P, P, 128, ULY_BF16, 0, sh.get(), nullptr) == ULY_OK,
           "unpack_qkv ok");
    expect(g_launches == before + 6, "valid permutes reach the launchers");
    for (int nt = 1; nt <= 3; ++nt) {
      auto multi = ptrs(nt * P);
      auto outs = ptrs(nt);
      std::unique_ptr<int[]> H(new int[nt]);
      for (int i = 0; i < nt; ++i) H[i] = (i + 1) * P;
      expect(ulysses_pack_multi(nt, multi.get(), H.get(), P, 32, 128, ULY_BF16, 0, outs.get(), nullptr) == ULY_OK,
             "pack_multi ok");
      expect(ulysses_unpack_multi(nt, outs.get(), H.get(), P, 32, 128, ULY_BF16, 0, multi.get(), nullptr) == ULY_OK,
             "unpack_multi ok");
    }
  }
  auto sh = ptrs(4);
  const int before = g_launches;
  expect(ulysses_pack(sh.get(), 0, 256, 8, 64, ULY_BF16, 0, fake(9), nullptr) == ULY_ERR_INVALID_ARG, "P=0");
  expect(ulysses_pack(sh.get(), 4, 256, 6, 64, ULY_BF16, 0, fake(9), nullptr) == ULY_ERR_INVALID_ARG, "H%P");
  expect(ulysses_pack(sh.get(), 4, 256, 8, 96, ULY_BF16, 0, fake(9), nullptr) == ULY_ERR_INVALID_ARG, "D=96");
  expect(ulysses_pack(sh.get(), 4, 256, 8, 64, (uly_dtype)7, 0, fake(9), nullptr) == ULY_ERR_INVALID_ARG, "dtype");
  expect(ulysses_pack(sh.get(), 4, 256, 8, 64, ULY_BF16, 4, fake(9), nullptr) == ULY_ERR_INVALID_ARG, "group");
  expect(ulysses_pack(nullptr, 4, 256, 8, 64, ULY_BF16, 0, fake(9), nullptr) == ULY_ERR_INVALID_ARG, "NULL shards");
  sh[2] = nullptr;
  expect(ulysses_unpack(fake(9), 4, 256, 8, 64, ULY_BF16, 0, sh.get(), nullptr) == ULY_ERR_INVALID_ARG, "NULL shard");
  expect(g_launches == before, "invalid permutes launch nothing");
  expect(std::strstr(uly_last_error(), "shards[2]") != nullptr, "message names the shard");
}

void attention() {
  const int before = g_launches;
  std::vector<int32_t> cu_host = {0, 100, 100, 300};
  const int32_t* cu = reinterpret_cast<const int32_t*>(fake(50));
  for (uly_dtype dt : {ULY_BF16, ULY_F32})
    for (int D : {64, 128}) {
      expect(attn_fwd(fake(1), fake(2), fake(3), fake(4), (float*)fake(5), 300, 4, 1, D, dt, cu, 3, 0.1f, 1,
                      nullptr) == ULY_OK, "fwd ok");
      size_t ws = 0;
      expect(attn_bwd_workspace_size(300, 4, 1, D, dt, &ws) == ULY_OK && ws > 0, "ws size");
      expect(attn_bwd(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), fake(7), fake(8), fake(9), 300,
                      4, 1, D, dt, cu, 3, 0.1f, 0, fake(10), ws, nullptr) == ULY_OK, "bwd ok");
      expect(attn_bwd_ex(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), fake(7), fake(8), fake(9), 300,
                         4, 1, D, dt, nullptr, 0, 0.1f, 1, fake(10), ws, nullptr, ULY_F32) == ULY_OK, "bwd_ex ok");
      expect(attn_bwd_accumulate(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), fake(7), fake(8),
                                 fake(9), 300, 4, 1, D, dt, nullptr, 0, 0.1f, 1, fake(10), ws, nullptr) == ULY_OK,
             "bwd_accumulate ok");
      expect(attn_bwd_noalloc(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), fake(7), fake(8), fake(9),
                              300, 4, 1, D, dt, nullptr, 0, 0.1f, 1, nullptr) == ULY_OK, "bwd_noalloc ok");
      expect(attn_bwd(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), fake(7), fake(8), fake(9), 300,
                      4, 1, D, dt, cu, 3, 0.1f, 1, fake(10), ws - 1, nullptr) == ULY_ERR_INVALID_ARG,
             "bwd workspace too small");
    }
  for (int P : {1, 8}) {
    auto q = ptrs(P), k = ptrs(P), v = ptrs(P);
    expect(attn_fwd_from_shards(q.get(), k.get(), v.get(), P, 128, 4 * P, P, 128, ULY_BF16, 0, fake(1),
                                (float*)fake(2), nullptr, 0, 0.1f, 1, nullptr) == ULY_OK, "fwd_from_shards ok");
  }
  for (int n : {1, 3, 64}) {
    auto o = ptrs(n), l = ptrs(n);
    expect(attn_merge(o.get(), (const float* const*)l.get(), n, 100, 4, 128, ULY_BF16, fake(200), (float*)fake(201),
                      nullptr) == ULY_OK, "merge ok");
  }
  const int valid = g_launches;
  expect(attn_fwd(fake(1), fake(2), fake(3), fake(4), (float*)fake(5), 300, 4, 3, 128, ULY_BF16, nullptr, 0, 0.1f, 1,
                  nullptr) == ULY_ERR_INVALID_ARG, "fwd hq%hk");
  expect(attn_fwd(fake(1), fake(2), fake(3), fake(4), (float*)fake(5), 300, 4, 1, 128, ULY_BF16, nullptr, 0, -1.f, 1,
                  nullptr) == ULY_ERR_INVALID_ARG, "fwd scale");
  expect(attn_bwd_ex(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), fake(7), fake(8), fake(9), 300, 4,
                     1, 128, ULY_F32, nullptr, 0, 0.1f, 1, fake(10), 1 << 30, nullptr, ULY_BF16) ==
             ULY_ERR_UNSUPPORTED, "bwd_ex grad_dt");
  expect(attn_bwd_noalloc(fake(1), fake(2), fake(3), fake(4), fake(5), (float*)fake(6), fake(7), fake(8), fake(9),
                          51781, 4, 1, 128, ULY_BF16, nullptr, 0, 0.1f, 1, nullptr) == ULY_ERR_UNSUPPORTED,
         "noalloc too large");
  expect(g_launches == valid, "invalid attention calls launch nothing");
  expect(g_launches > before, "valid attention calls reach the launchers");
  // host check of document offsets on exactly sized arrays
  std::unique_ptr<int32_t[]> a(new int32_t[4]{0, 100, 100, 300});
  expect(uly_check_cu_seqlens(a.get(), 3, 300) == ULY_OK, "cu ok");
  expect(uly_check_cu_seqlens(a.get(), 3, 299) == ULY_ERR_INVALID_ARG, "cu last != N");
  a[2] = 400;
  expect(uly_check_cu_seqlens(a.get(), 3, 300) == ULY_ERR_INVALID_ARG, "cu beyond N");
  expect(uly_check_cu_seqlens(a.get(), 0, 300) == ULY_ERR_INVALID_ARG, "cu ndocs 0");
  expect(uly_check_cu_seqlens(nullptr, 3, 300) == ULY_ERR_INVALID_ARG, "cu NULL");
}

void thread_local_messages() {
  ulysses_pack(nullptr, 0, 1, 1, 64, ULY_BF16, 0, fake(), nullptr);
  const std::string mine = uly_last_error();
  std::string theirs;
  std::thread t([&] {
    theirs = uly_last_error();  // nothing failed on this thread yet
    ulysses_pack(nullptr, 2, 1, 2, 96, ULY_BF16, 0, fake(), nullptr);
  });
  t.join();
  expect(theirs.empty(), "a new thread starts with an empty message");
  expect(mine == uly_last_error(), "another thread's failure leaves this thread's message");
}

}  // namespace

int main() {
  permutes();
  attention();
  thread_local_messages();
  if (g_fail) {
    std::fprintf(stderr, "%d of %d checks failed\n", g_fail, g_checks);
    return 1;
  }
  std::printf("ok %d\n", g_checks);
  return 0;
}
