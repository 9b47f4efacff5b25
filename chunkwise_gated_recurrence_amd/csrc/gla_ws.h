// gla_ws.h -- the 256-byte header at the start of every libgtrgla workspace.
//
// Word 0 is the error word: sticky bits set by kernels (never cleared by a
// kernel), read and cleared by gtr_gla_workspace_status. Words 1-3 describe
// what the rest of the workspace holds, so that a fused launch can tell a
// workspace it may trust (zeroed by the library, or last used by fused launches
// of the same exchange layout) from one it may not (anything else).
#pragma once

namespace gtrgla {

constexpr int kWsHeaderBytes = 256;
constexpr int kWsErrWord = 0;       // error bits, below
constexpr int kWsMagicWord = 1;     // kWsClean, kWsFused or kWsDirty (anything else: unknown)
constexpr int kWsLayoutWord = 2;    // exchange layout of the fused launches that use it
constexpr int kWsLayoutCheck = 3;   // ~layout

constexpr unsigned int kWsClean = 0x4E454C43u;   // zeroed by the library, no layout yet
constexpr unsigned int kWsFused = 0x31414C47u;   // exchange words of the layout in word 2
constexpr unsigned int kWsDirty = 0x59545244u;   // written by other kernels (generic path)

constexpr unsigned int kWsErrExchange = 1u;      // an exchange wait gave up (outputs NaN)
constexpr unsigned int kWsErrState = 2u;         // launched on an untrusted workspace (outputs NaN)

}  // namespace gtrgla
