// Recorded launches of the host-only build (see stub_launchers.cpp).
#pragma once

#include "../../exact_io_aware_30_amd/csrc/fa_launch.h"

namespace fa {

struct Record {
  char kind = 0;   // 'F' forward, 'P' pre-pass, 'K' dK/dV, 0 none
  char kind2 = 0;  // 'Q' when a dQ launch followed
  FwdArgs fwd{};
  PreArgs pre{};
  BwdArgs bwd{};
  BwdArgs bwd_dq{};
};

extern Record g_last;
extern int g_launches;

}  // namespace fa
