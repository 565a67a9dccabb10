// Launch side of the chunk-parallel forward pass for Falcon-3 / 3A with a
// window of 2, 4 or 8 pairs (kernels in split_impl.h): systems of 64 virtual
// rows, i.e. 64 / Bw steps each.
#include "split_impl.h"

namespace falcon {

namespace {

// Compile-time dispatch over (variant, dtype, d, window) for chunk 64: `fn`
// receives the variant, a null pointer of the input type, d and the window as
// compile-time values; unlisted combinations return a value-initialised result.
template <typename Fn>
auto dispatch_win(int variant, bool bf16, int d, int chunk, int window, Fn &&fn) -> decltype(fn(std::integral_constant<int, V_F3>(), (float *)nullptr, std::integral_constant<int, 32>(), std::integral_constant<int, 2>())) {
  using R = decltype(fn(std::integral_constant<int, V_F3>(), (float *)nullptr, std::integral_constant<int, 32>(), std::integral_constant<int, 2>()));
  if (chunk != 64) return R();
  auto by_w = [&](auto v, auto *t, auto dd) -> R {
    switch (window) {
      case 2: return fn(v, t, dd, std::integral_constant<int, 2>());
      case 4: return fn(v, t, dd, std::integral_constant<int, 4>());
      case 8: return fn(v, t, dd, std::integral_constant<int, 8>());
    }
    return R();
  };
  auto by_d = [&](auto v, auto *t) -> R {
    if (d == 32) return by_w(v, t, std::integral_constant<int, 32>());
    if (d == 64) return by_w(v, t, std::integral_constant<int, 64>());
    if constexpr (sizeof(*t) == 2) {
      if (d == 128) return by_w(v, t, std::integral_constant<int, 128>());
    }
    return R();
  };
  auto by_type = [&](auto v) -> R {
    if (bf16) return by_d(v, (__bf16 *)nullptr);
    return by_d(v, (float *)nullptr);
  };
  switch (variant) {
    case V_F3: return by_type(std::integral_constant<int, V_F3>());
    case V_F3A: return by_type(std::integral_constant<int, V_F3A>());
  }
  return R();
}

}  // namespace

bool chunk_fwd_split_win_supported(int variant, bool bf16, int d, int chunk, int window) {
  return dispatch_win(variant, bf16, d, chunk, window, [](auto v, auto *t, auto dd, auto w) -> bool {
    using IT = std::remove_pointer_t<decltype(t)>;
    return pick_ns<decltype(v)::value, IT, decltype(dd)::value, 64, decltype(w)::value>(1) > 0;
  });
}

size_t chunk_fwd_split_win_workspace(int variant, bool bf16, int d, int chunk, int window, int bh, int T) {
  return dispatch_win(variant, bf16, d, chunk, window, [bh, T](auto v, auto *t, auto dd, auto w) -> size_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return Split<decltype(v)::value, IT, decltype(dd)::value, 64, decltype(w)::value>::workspace(bh, T);
  });
}

size_t chunk_fwd_split_win_workspace_varlen(int variant, bool bf16, int d, int chunk, int window, int N, int H,
                                            int total) {
  return dispatch_win(variant, bf16, d, chunk, window, [N, H, total](auto v, auto *t, auto dd, auto w) -> size_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return Split<decltype(v)::value, IT, decltype(dd)::value, 64, decltype(w)::value>::workspace_varlen(N, H, total);
  });
}

hipError_t launch_chunk_fwd_split_win(int variant, bool bf16, int d, int chunk, int window, const FwdArgs &a,
                                      void *ws, hipStream_t st) {
  if (!chunk_fwd_split_win_supported(variant, bf16, d, chunk, window)) return hipErrorInvalidValue;
  return dispatch_win(variant, bf16, d, chunk, window, [&](auto v, auto *t, auto dd, auto w) -> hipError_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return launch_split<decltype(v)::value, IT, decltype(dd)::value, 64, decltype(w)::value>(a, ws, st);
  });
}

int chunk_fwd_onepass_win_ns(int variant, bool bf16, int d, int chunk, int window, int bh) {
  return dispatch_win(variant, bf16, d, chunk, window, [bh](auto v, auto *t, auto dd, auto w) -> int {
    using IT = std::remove_pointer_t<decltype(t)>;
    return pick_ns<decltype(v)::value, IT, decltype(dd)::value, 64, decltype(w)::value, true>(bh);
  });
}

hipError_t launch_chunk_fwd_onepass_win(int variant, bool bf16, int d, int chunk, int window, const FwdArgs &a,
                                        hipStream_t st) {
  return dispatch_win(variant, bf16, d, chunk, window, [&](auto v, auto *t, auto dd, auto w) -> hipError_t {
    using IT = std::remove_pointer_t<decltype(t)>;
    return launch_onepass<decltype(v)::value, IT, decltype(dd)::value, 64, decltype(w)::value>(a, st);
  });
}

}  // namespace falcon
